// libpagedattn -- HIP kernels for gfx950 (MI355X) and the C entry points.
//
// Kernels:
//   reshape_and_cache_kernel   scatter new K/V rows into the paged cache by
//                              slot_mapping ("FlashAttention 在 vLLM 中的实现分析",
//                              sections 4.2 and 8.2)
//   attn_small_kernel<D>       paged attention for work items of <= 16 rows
//                              (decode: one token x the G query heads of a KV
//                              head), bound by HBM reads of K/V
//   attn_tiled_kernel<D>       paged attention for 128-row blocks (prefill),
//                              bound by the matrix cores
//   attn_tiled_wide_kernel<D>  the same for 256-row blocks: 8 waves share
//                              each K/V tile (long prefills, D <= 128)
//   attn_mixed_kernel<D>       small-row and 128-row items in one launch
//   attn_mixed_dma_kernel<128> the same for a bf16 cache with a power-of-two
//                              block size, its 128-row items loading K/V
//                              tiles into LDS by DMA (tiled_dma4_body)
//   attn_tiled_dma4_kernel<128> 128-row items alone, by tiled_dma4_body
//                              (every tiled-only launch of a bf16 cache at
//                              D = 128 with a power-of-two block size)
//   split_reduce_kernel<D>     LSE merge of split-KV partials (section 1.3
//                              num_splits)
//   merge_states_kernel        two-way LSE merge (section 6.3, step 3)
//
// Both attention kernels compute S^T = K Q^T and O^T = V^T P^T with bf16
// MFMA and fp32 accumulation, so that every lane owns one query row: its
// running max, its row sum and its slice of O^T never leave the lane except
// for one cross-lane max/sum between the lanes that split the row's keys.
// K is read from memory in its natural [key][d] layout as the A operand of
// the first product; V is staged row-major in LDS and read back transposed
// with ds_read_b64_tr_b16, which hands each lane four keys of one d column.
// The softmax works in the log2 domain (scores pre-multiplied by
// scale*log2(e), exp2), and converts the LSE to natural log on output.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pagedattn.h"
#include "plan_internal.h"

namespace {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16x8_t pack_bf16x8(const float* p) {
  uint4 w;
  w.x = pack_bf16x2(p[0], p[1]);
  w.y = pack_bf16x2(p[2], p[3]);
  w.z = pack_bf16x2(p[4], p[5]);
  w.w = pack_bf16x2(p[6], p[7]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// acc + the sum of the bf16 values packed in w (v_dot2 with ones: the bf16
// values are exact in fp32, so this sums exactly the probabilities that the
// PV product multiplies)
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                          __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}
__device__ __forceinline__ float add_bf16x8(bf16x8_t p, float acc) {
  const u32x4_t w = __builtin_bit_cast(u32x4_t, p);
  return add_bf16x2(w[3], add_bf16x2(w[2], add_bf16x2(w[1], add_bf16x2(w[0], acc))));
}

// 16 E4M3 codes (one 16-byte load) -> 16 bf16 values in two 16-byte chunks.
// Exact: every E4M3 value is a bf16 value, and the conversion scale is 1.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ void e4m3x16_to_bf16(u32x4_t w, u32x4_t& lo, u32x4_t& hi) {
  lo = u32x4_t{e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
               e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
  hi = u32x4_t{e4m3x2_to_bf16x2<false>(w[2]), e4m3x2_to_bf16x2<true>(w[2]),
               e4m3x2_to_bf16x2<false>(w[3]), e4m3x2_to_bf16x2<true>(w[3])};
}

// fp32 -> E4M3 code (OCP E4M3: bias 7, subnormals, S.1111.111 = NaN, largest
// finite 448): nearest value, ties to the even code, saturating at +-448,
// NaN -> 0x7F.  Written out in integer steps so that the result does not
// depend on a conversion instruction's rounding or clamping mode.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;               // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;       // |x| >= 448, infinities: saturate
  if (a < 0x3c800000u) {                           // |x| < 2^-6: multiples of 2^-9
    const float f = __builtin_bit_cast(float, a) * 512.0f;   // exact
    return sign | (uint32_t)__builtin_rintf(f);    // round half to even; 8 = 2^-6
  }
  const uint32_t e = (a >> 23) - 127u + 7u;        // biased E4M3 exponent, 1..15
  const uint32_t mant = a & 0x7fffffu;
  uint32_t q = mant >> 20;
  const uint32_t rem = mant & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;   // q = 8 carries
  const uint32_t code = (e << 3) + q;
  return sign | (code > 0x7eu ? 0x7eu : code);
}

__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8_t zero8() {
  bf16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
  return z;
}

// transposing LDS read: within each 16-lane group, lane r receives element
// r%4 of the 8-byte rows addressed by lanes r/4, r/4+4, r/4+8, r/4+12
__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t cat(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The values of lanes l and l ^ 16 (v_permlane16_swap) or l and l ^ 32
// (v_permlane32_swap), in lane order: a VALU exchange with no LDS traffic
// or wait.  max and a two-term sum of the pair equal those of l and its
// partner exactly.
template <int X>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  static_assert(X == 16 || X == 32, "lane_pair");
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  uint32_t r0, r1;
  if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
template <int X>
__device__ __forceinline__ float max_xor(float v) {
  float a, b;
  lane_pair<X>(v, a, b);
  return fmaxf(a, b);
}
template <int X>
__device__ __forceinline__ float sum_xor(float v) {
  float a, b;
  lane_pair<X>(v, a, b);
  return a + b;
}

// Load of a wave-uniform int32 from memory that no kernel of the launch
// writes (work list, lengths, block table): through the constant address
// space, so it becomes a scalar load instead of a vector load whose wait
// would also wait for every prefetch in flight.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p) {
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  return *(const_i32_ptr)(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ float ld_uniform(const float* p) {
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  return *(const_f32_ptr)(reinterpret_cast<uintptr_t>(p));
}

struct Item {
  int seq, kvh, row0, nrows, kv0, kv1, prow;
  int t0;     // the sequence's first query token
  int koff;   // Lk - Lq: query i's last visible key under the causal mask is i + koff
};

__device__ __forceinline__ Item load_item(const int32_t* p) {
  Item it;
  it.seq = ld_uniform(p + 0);
  it.kvh = ld_uniform(p + 1);
  it.row0 = ld_uniform(p + 2);
  it.nrows = ld_uniform(p + 3);
  it.kv0 = ld_uniform(p + 4);
  it.kv1 = ld_uniform(p + 5);
  it.prow = ld_uniform(p + 6);
  it.t0 = ld_uniform(p + 8);
  it.koff = ld_uniform(p + 9);
  return it;
}

struct AttnArgs {
  const int32_t* items;
  const uint16_t* q;
  const uint16_t* cache;
  const int32_t* cu;
  const int32_t* seqused_k;
  const int32_t* block_table;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int64_t plane;      // elements in one cache plane (NB*BS*Hkv*D)
  int H, Hkv, G, BS, MB, bt_stride, causal;
  int NB;             // physical blocks: a block-table entry outside [0, NB) reads as zeros
  int bs_log2;        // log2(BS) when BS is a power of two, else -1
  float scale_log2;   // scale * log2(e)
  const float* k_scale;   // E4M3 cache: per-KV-head dequantisation scales
  const float* v_scale;
  const float* s_aux;     // per-query-head sink logits, or null
  int window;             // sliding window W (0: none)
};

// The sink's share of the denominator, added where a row's final state is
// formed (never to split partials: their merge adds it once).  m: the row's
// reference max, l / lr: its sums relative to m, all in the log2 domain.
// Returns the factor that rescales O (relative to m) and replaces m, l, lr
// by the sink-inclusive values relative to the new reference.
__device__ __forceinline__ float add_sink(float sink_l2, float& m, float& l, float& lr) {
  const float M = fmaxf(m, sink_l2);
  const float a = (m == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m - M);
  const float b = __builtin_amdgcn_exp2f(sink_l2 - M);
  m = M;
  l = l * a + b;
  lr = lr * a + b;
  return a;
}

// 64-bit load of a wave-uniform value (the token's slot) as a scalar load
__device__ __forceinline__ int64_t ld_uniform64(const int64_t* p) {
  typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;
  return *(const_i64_ptr)(reinterpret_cast<uintptr_t>(p));
}

// ---------------------------------------------------------------------------
// reshape_and_cache: one wave per RC_TOKENS_PER_WAVE consecutive tokens (four
// waves per workgroup).  The lanes walk each token's K row and V row in
// 16-byte chunks, two chunks per plane per token, so no index needs a
// division.  The source rows do not depend on the slots, so every load of
// the wave's tokens is issued before the first slot is tested: one memory
// latency per wave, not two.  Slots outside [0, num_slots) are skipped.  Two
// tokens per wave halve the workgroup count, so that a batch of a few
// thousand tokens is one round of resident workgroups with no short second
// round at the end.
// ---------------------------------------------------------------------------
constexpr int RC_TOKENS_PER_WAVE = 2;

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value, int64_t key_stride,
    int64_t value_stride, uint16_t* __restrict__ cache, const int64_t* __restrict__ slot_mapping,
    int32_t num_tokens, int32_t cpr, int64_t row_elems, int64_t plane, int64_t num_slots) {
  constexpr int TPW = RC_TOKENS_PER_WAVE;
  const int t0 = __builtin_amdgcn_readfirstlane((blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW);
  if (t0 >= num_tokens) return;
  const int lane = threadIdx.x & 63;
  const int row_bytes = (int)(row_elems * 2);
  for (int c = lane; c < cpr; c += 128) {
    // chunk c and chunk c + 64 of each row; a lane without a second chunk
    // moves its first one twice
    const int c1 = c + 64 < cpr ? c + 64 : c;
    u32x4_t k[TPW][2], v[TPW][2];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = min(t0 + i, num_tokens - 1);     // a past-the-end token re-reads the last
      const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(key + (int64_t)t * key_stride);
      const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(value + (int64_t)t * value_stride);
      k[i][0] = __builtin_nontemporal_load(ks + c);
      v[i][0] = __builtin_nontemporal_load(vs + c);
      k[i][1] = __builtin_nontemporal_load(ks + c1);
      v[i][1] = __builtin_nontemporal_load(vs + c1);
    }
    // each token's destination rows as buffer resources, set up once the rows
    // are requested (the slot loads overlap them; the empty asm keeps the
    // compiler from hoisting them above the row loads): a token past the end
    // or with a skipped slot gets 0 records, so its stores are dropped and
    // the loop holds no branch (the compiler would otherwise sink the loads
    // into it)
    const int64_t* sm = slot_mapping;
    asm volatile("" : "+s"(sm));
    __amdgpu_buffer_rsrc_t kr[TPW], vr[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t slot = ld_uniform64(sm + min(t0 + i, num_tokens - 1));
      const bool ok = (t0 + i < num_tokens) & (slot >= 0) & (slot < num_slots);
      const int64_t off = (slot * row_elems) & -(int64_t)ok;
      kr[i] = __builtin_amdgcn_make_buffer_rsrc(cache + off, 0, row_bytes & -(int)ok, 0x00020000);
      vr[i] = __builtin_amdgcn_make_buffer_rsrc(cache + plane + off, 0, row_bytes & -(int)ok,
                                                0x00020000);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      __builtin_amdgcn_raw_buffer_store_b128(k[i][0], kr[i], 16 * c, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(v[i][0], vr[i], 16 * c, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(k[i][1], kr[i], 16 * c1, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(v[i][1], vr[i], 16 * c1, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Work-list upload: thread i copies words [4i, 4i + 4) (the last thread the
// remainder) from pinned host memory, read over the bus by the kernel itself.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void upload_words_kernel(const int32_t* __restrict__ src,
                                                           int32_t* __restrict__ dst,
                                                           int64_t n_words) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t w = 4 * i;
  if (w + 4 <= n_words) {
    reinterpret_cast<u32x4_t*>(dst)[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(src) + i);
  } else {
    for (int64_t k = w; k < n_words; ++k) dst[k] = src[k];
  }
}

// ---------------------------------------------------------------------------
// reshape_and_cache into an E4M3 cache: one wave per token, as above; a lane
// turns 16 elements of the K (V) row into 16 output bytes, code =
// E4M3(x / scale[kv head]), the division in IEEE fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 e4m3x16_from_bf16(const uint16_t* src, float sc) {
  const uint4 w0 = reinterpret_cast<const uint4*>(src)[0];
  const uint4 w1 = reinterpret_cast<const uint4*>(src)[1];
  const uint32_t in[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t bits = (k & 1) ? (in[k >> 1] & 0xffff0000u) : (in[k >> 1] << 16);
    o[k >> 2] |= f32_to_e4m3(__builtin_bit_cast(float, bits) / sc) << (8 * (k & 3));
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value, int64_t key_stride,
    int64_t value_stride, uint8_t* __restrict__ cache, const int64_t* __restrict__ slot_mapping,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int32_t num_tokens,
    int32_t cpr, int32_t chunks_per_head, int64_t row_elems, int64_t plane, int64_t num_slots) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= num_tokens) return;
  const int64_t slot = ld_uniform64(slot_mapping + t);
  if (slot < 0 || slot >= num_slots) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* ks = key + (int64_t)t * key_stride;
  const uint16_t* vs = value + (int64_t)t * value_stride;
  uint4* kd = reinterpret_cast<uint4*>(cache + slot * row_elems);
  uint4* vd = reinterpret_cast<uint4*>(cache + plane + slot * row_elems);
  for (int c = lane; c < cpr; c += 64) {
    const int h = c / chunks_per_head;
    kd[c] = e4m3x16_from_bf16(ks + c * 16, k_scale[h]);
    vd[c] = e4m3x16_from_bf16(vs + c * 16, v_scale[h]);
  }
}

// ---------------------------------------------------------------------------
// Small-row attention: one workgroup of 4 waves per work item of <= 16 rows
// (decode: the G query heads of one KV head, times at most 16/G tokens).
// The item's key range is walked in 16-key steps; wave w takes steps w,
// w+4, w+8, ...  K and V are read once, so the kernel is bound by HBM:
//   * loads are non-temporal and coalesced: CPR = D/8 consecutive lanes read
//     one key row (D*2 contiguous bytes) 16 bytes each, so every wave
//     instruction covers 64/CPR whole rows;
//   * each wave keeps PF steps of loads in flight in registers, and stages
//     the step it computes in a private LDS tile (K and V, [16][D]) whose
//     16-byte chunks are XOR-swizzled by row so that the MFMA operand reads
//     (four lanes per row for K, a transposing read for V) avoid bank
//     conflicts.
// Lane (n = lane%16, g = lane/16) owns query row n: S^T = K Q^T on
// 16x16x32 MFMA (k-step t: d chunk 4t+g), O^T = V^T P^T on 16x16x16 MFMA
// (P^T slots = keys 4g..4g+3, exactly where the S^T layout left them).
// Item key ranges start on a multiple of 16, and block_size is a multiple
// of 16, so the 16 keys of a step lie in one cache block.
// ---------------------------------------------------------------------------

template <int D>
struct SmallCfg {
  static constexpr int CPR = D / 8;          // 16-byte chunks per key row
  static constexpr int LPR = 64 / CPR;       // key rows per wave load instruction
  static constexpr int NLD = 16 / LPR;       // load instructions per plane per step
  // steps of loads in flight per wave at 2 waves per SIMD (the mixed
  // kernel); the small-row kernel runs D = 128 with two steps, which fits
  // the registers of 3 waves per SIMD (4 with an E4M3 cache): as many bytes
  // in flight per compute unit, and a third (fourth) workgroup covers
  // another's start-up
  static constexpr int PF = (D == 256) ? 2 : 3;
  static constexpr int PF_SMALL = (D >= 128) ? 2 : 3;
  static constexpr int RB = D * 2;           // bytes per LDS row
  static constexpr int WAVE_LDS = 2 * 16 * RB;
  // floats per row of the epilogue's merge area: the 4-float pad puts the
  // 16 rows of a 16-byte store or load in different banks
  static constexpr int SD = D + 4;
};

// chunk position of (row r, chunk c) inside an LDS row
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ ((r % (CPR / 2)) * 2);
}

// LDS bytes of one small-row workgroup: four staging tiles, or the epilogue
// merge area
template <int D>
constexpr int small_lds_bytes() {
  return (4 * SmallCfg<D>::WAVE_LDS > (4 * 16 * SmallCfg<D>::SD + 3 * 64) * 4)
             ? 4 * SmallCfg<D>::WAVE_LDS
             : (4 * 16 * SmallCfg<D>::SD + 3 * 64) * 4;
}

// loads of one key row: D*ES bytes in 16-byte chunks (ES = 1 for an E4M3
// cache, whose 16-byte chunk becomes two bf16 chunks in LDS)
template <int D, bool FP8>
struct SmallLoad {
  static constexpr int ES = FP8 ? 1 : 2;
  static constexpr int CPR = D * ES / 16;    // 16-byte chunks per key row
  static constexpr int LPR = 64 / CPR;       // key rows per wave load instruction
  static constexpr int NLD = 16 / LPR;       // load instructions per plane per step
};

template <int D, bool FP8, int PF>
__device__ __forceinline__ void small_body(const AttnArgs& a, const int32_t* item, uint8_t* smem) {
  using C = SmallCfg<D>;
  using LD = SmallLoad<D, FP8>;
  constexpr int CPR = C::CPR, RB = C::RB;
  constexpr int LPR = LD::LPR, NLD = LD::NLD, ES = LD::ES;
  constexpr int NT = D / 32;        // QK k-steps
  constexpr int NDT = D / 16;       // 16-wide d tiles of O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = lane & 15, g = lane >> 4;
  const Item it = load_item(item);
  // the item carries the sequence's first token and causal offset, and its
  // rows and key range are already clipped to the sequence
  const int t0 = it.t0;
  const int G = a.G;
  const int nrows = it.nrows;
  const int kv1 = min(it.kv1, a.MB * a.BS);
  const int kv0 = it.kv0;

  const int r = it.row0 + n;
  const bool row_ok = n < nrows;
  const int tok = r / G;
  const int head = it.kvh * G + (r - tok * G);
  const int row_limit = a.causal ? tok + it.koff : INT_MAX;
  const int row_lo = a.window > 0 ? tok + it.koff - (a.window - 1) : INT_MIN;
  // an E4M3 cache holds K / k_scale and V / v_scale of each KV head: the
  // scores take k_scale inside the exponent's factor, O takes v_scale at the end
  const float sl2 = FP8 ? a.scale_log2 * ld_uniform(a.k_scale + it.kvh) : a.scale_log2;
  const float vsc = FP8 ? ld_uniform(a.v_scale + it.kvh) : 1.f;

  // Q^T operand: k-step t, slot j <-> d = 32t + 8g + j
  bf16x8_t qf[NT];
  if (row_ok) {
    const uint16_t* qp = a.q + ((int64_t)(t0 + tok) * a.H + head) * D + 8 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t) qf[t] = ld16(qp + 32 * t);
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) qf[t] = zero8();
  }

  // loader geometry: this lane reads chunk lc of rows lr + LPR*i
  const int lr = lane / LD::CPR, lc = lane % LD::CPR;
  const int64_t row_elems = (int64_t)a.Hkv * D;
  const int32_t* btrow = a.block_table + (int64_t)it.seq * a.bt_stride;
  uint8_t* wl = smem + wave * C::WAVE_LDS;       // K rows [0,16), V rows [16,32)
  // chunk position in LDS.  An E4M3 lane widens one 16-byte code chunk into
  // bf16 chunks 2c and 2c+1 and stores them with two instructions, and 8
  // lanes (one key row at D >= 128) share an LDS pass of 128 bytes: with the
  // two halves of code chunks 4..7 of every 8 trading places, each pass of
  // each store covers the 8 bank groups once (measured: 4.5 M conflict
  // cycles per launch without).  Readers see a uniform permutation of the
  // chunks they read.
  auto sw = [](int r, int c) {
    return swz<CPR>(r, (FP8 && D >= 128) ? (c ^ ((c >> 3) & 1)) : c);
  };

  const int nsteps = (kv1 > kv0 + wave * 16) ? (kv1 - kv0 - wave * 16 + 63) / 64 : 0;

  u32x4_t buf[PF][2 * NLD];
  // buffer loads: a step's rows past the key range (and steps past the
  // range) read as zero without touching memory, so every step issues the
  // same loads and the wait before each step counts exactly the later steps'
  // loads still in flight
  const int64_t kv_bytes = (int64_t)it.kvh * D * ES;
  int voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) voff[i] = (lr + LPR * i) * (int)(row_elems * ES) + lc * 16;
  const uint8_t* cache_b = reinterpret_cast<const uint8_t*>(a.cache);
  auto issue = [&](u32x4_t* bf, int st) {
    const int kb = kv0 + 16 * (wave + 4 * st);
    int nrec = 0;
    int64_t boff = 0;
    if (kb < kv1) {
      const int blk = (a.bs_log2 >= 0) ? (kb >> a.bs_log2) : (kb / a.BS);
      const int phys = ld_uniform(btrow + blk);
      if ((unsigned)phys < (unsigned)a.NB) {
        const int valid = min(16, kv1 - kb);
        boff = ((int64_t)phys * a.BS + (kb - blk * a.BS)) * row_elems * ES + kv_bytes;
        nrec = (valid - 1) * (int)(row_elems * ES) + D * ES;
      }
    }
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cache_b + boff), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(cache_b + a.plane * ES + boff), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      bf[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, voff[i], 0, 2));
      bf[NLD + i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i], 0, 2));
    }
  };

  // l_run sums the fp32 probabilities (for the LSE), lr_run the bf16-rounded
  // ones that the PV product multiplies (for the normalisation of O)
  float m_run = kNegInf, l_run = 0.f, lr_run = 0.f;
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < PF; ++p) issue(buf[p], p);

  // LDS addresses that do not change between steps
  const int vr = 4 * g + (n >> 2);                         // V row of this lane's transposing read
  for (int it0 = 0; it0 < nsteps; it0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int st = it0 + p;
      if (st >= nsteps) break;
      // stage step st (swizzled) in this wave's LDS tile
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = lr + LPR * i;
        if constexpr (FP8) {
          u32x4_t k0, k1, v0, v1;
          e4m3x16_to_bf16(buf[p][i], k0, k1);
          e4m3x16_to_bf16(buf[p][NLD + i], v0, v1);
          *reinterpret_cast<u32x4_t*>(wl + row * RB + sw(row, 2 * lc) * 16) = k0;
          *reinterpret_cast<u32x4_t*>(wl + row * RB + sw(row, 2 * lc + 1) * 16) = k1;
          *reinterpret_cast<u32x4_t*>(wl + (16 + row) * RB + sw(row, 2 * lc) * 16) = v0;
          *reinterpret_cast<u32x4_t*>(wl + (16 + row) * RB + sw(row, 2 * lc + 1) * 16) = v1;
        } else {
          *reinterpret_cast<u32x4_t*>(wl + row * RB + sw(row, lc) * 16) = buf[p][i];
          *reinterpret_cast<u32x4_t*>(wl + (16 + row) * RB + sw(row, lc) * 16) = buf[p][NLD + i];
        }
      }
      issue(buf[p], st + PF);
      const int kb = kv0 + 16 * (wave + 4 * st);

      // S^T (16 keys x 16 rows): lane (n, g) reg i <- key kb + 4g + i
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8_t ka =
            *reinterpret_cast<const bf16x8_t*>(wl + n * RB + sw(n, 4 * t + g) * 16);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[t], s, 0, 0, 0);
      }
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 4 * g + i;
        x[i] = (key >= kv1 || key > row_limit || key < row_lo) ? kNegInf : s[i] * sl2;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = max_xor<16>(mx);
      mx = max_xor<32>(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
      l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m_run = m_new;
      // rescale O only when some row's running max moved
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      }
      uint2 pw;
      pw.x = pack_bf16x2(pr[0], pr[1]);
      pw.y = pack_bf16x2(pr[2], pr[3]);
      lr_run = add_bf16x2(pw.y, add_bf16x2(pw.x, lr_run * alpha));
      const bf16x4_t pb = __builtin_bit_cast(bf16x4_t, pw);
      // O^T += V^T P^T; lane (s, g) of each 16-lane group reads 4 d of key
      // 4g + s/4, so lane s receives d = 16dt + s of keys 4g..4g+3
      const uint8_t* vrow = wl + (16 + vr) * RB + 8 * (n & 1);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int chunk = 2 * dt + ((n & 3) >> 1);
        const bf16x4_t av = lds_read_tr(reinterpret_cast<const uint16_t*>(vrow + sw(vr, chunk) * 16));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, o[dt], 0, 0, 0);
      }
    }
  }

  // ---- merge the four waves' partial states through LDS
  l_run = sum_xor<32>(sum_xor<16>(l_run));
  lr_run = sum_xor<32>(sum_xor<16>(lr_run));
  __syncthreads();
  constexpr int SD = C::SD;
  float* so = reinterpret_cast<float*>(smem);
  float* sm = so + 4 * 16 * SD;
  float* sl = sm + 64;
  float* sr = sl + 64;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *reinterpret_cast<f32x4_t*>(so + (wave * 16 + n) * SD + 16 * dt + 4 * g) = o[dt];
  if (g == 0) {
    sm[wave * 16 + n] = m_run;
    sl[wave * 16 + n] = l_run;
    sr[wave * 16 + n] = lr_run;
  }
  __syncthreads();
  constexpr int DPT = D / 16;  // d elements per thread in the epilogue
  const int er = tid >> 4, ec = tid & 15;
  if (er < nrows) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w * 16 + er]);
    float wt[4], L = 0.f, Lr = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm[w * 16 + er];
      wt[w] = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += wt[w] * sl[w * 16 + er];
      Lr += wt[w] * sr[w * 16 + er];
    }
    const int rr = it.row0 + er;
    const int etok = rr / G;
    const int ehead = it.kvh * G + (rr - etok * G);
    float fo = 1.f;      // rescales the weighted O when a sink moves the reference
    if (a.s_aux && it.prow < 0) fo = add_sink(a.s_aux[ehead] * kLog2e, M, L, Lr);
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : vsc * fo / Lr;
    const float lse_v = empty ? kNegInf : (M + __log2f(L)) * kLn2;
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; e += 4) {
      f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        sum += wt[w] * *reinterpret_cast<const f32x4_t*>(so + (w * 16 + er) * SD + ec * DPT + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[e + k] = sum[k] * inv;
    }
    if (it.prow < 0) {
      const int64_t orow = (int64_t)(t0 + etok) * a.H + ehead;
      uint16_t* op = a.out + orow * D + ec * DPT;
      if constexpr (DPT % 8 == 0) {
#pragma unroll
        for (int e = 0; e < DPT; e += 8) *reinterpret_cast<bf16x8_t*>(op + e) = pack_bf16x8(acc + e);
      } else {
        static_assert(DPT == 4, "epilogue store");
        uint2 w;
        w.x = pack_bf16x2(acc[0], acc[1]);
        w.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2*>(op) = w;
      }
      if (ec == 0 && a.lse) a.lse[orow] = lse_v;
    } else {
      float* pp = a.part_o + (int64_t)(it.prow + er) * D + ec * DPT;
#pragma unroll
      for (int e = 0; e < DPT; e += 4)
        *reinterpret_cast<f32x4_t*>(pp + e) = f32x4_t{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
      if (ec == 0) a.part_lse[it.prow + er] = lse_v;
    }
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(256, (D <= 128 ? (FP8 ? 4 : 3) : 1)) void attn_small_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[small_lds_bytes<D>()];
  small_body<D, FP8, SmallCfg<D>::PF_SMALL>(a, a.items + (int64_t)blockIdx.x * PA_ITEM_WORDS, smem);
}

// ---------------------------------------------------------------------------
// Tiled attention: one workgroup of 4 waves per 128-row block (8 waves per
// 256-row block in the wide kernel); wave w owns rows 32w..32w+31 (lane
// (n = lane%32, h = lane/32) owns row n and the key half h of each 32x32
// MFMA tile).  Key tiles of 64 keys are gathered through the block table by
// threads 0..255 into registers one tile ahead (16 consecutive lanes per
// 256-byte key row, one bounds-checked buffer load per plane per 16 keys),
// then stored to LDS, where every wave of the workgroup reads them: K with a
// pitch of D+8 elements (conflict-free 16-byte operand reads), V with D+32
// (the transposing reads of two 16-lane groups cover all banks once).
//
// Online softmax with a lazy rescale: a row keeps its reference max until
// the tile max exceeds it by more than kRescaleSlack (log2 units), so the
// O accumulators are rescaled only when some row of the wave jumps.  The
// probabilities then stay below 2^kRescaleSlack, which bf16 and fp32
// represent with the same relative precision; the final normalisation uses
// the same reference, so the result is exact up to rounding.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.f;

template <bool B>
struct Bool {
  static constexpr bool value = B;
};

// LDS bytes of one tiled workgroup: two K tiles (pitch D+8) and two V tiles
// (pitch D+32) of 64 keys
template <int D>
constexpr int tiled_lds_bytes() {
  return 2 * 64 * (D + 8) * 2 + 2 * 64 * (D + 32) * 2;
}

// NW = 4: 128-row items; NW = 8: up to 256-row items, waves 0-3 load each
// tile and all 8 waves compute on it
template <int D, bool FP8, int NW = 4>
__device__ __forceinline__ void tiled_body(const AttnArgs& a, const int32_t* item, uint8_t* smem) {
  static_assert(NW == 4 || NW == 8, "tiled workgroup");
  constexpr int NKT = D / 16;       // QK k-steps (16 d each)
  constexpr int NDT = D / 32;       // 32-wide d tiles of O^T
  constexpr int KP = D + 8;
  constexpr int VP = D + 32;
  constexpr int CPR = D / 8;        // 16-byte chunks per key row
  constexpr int LOADS = 64 * CPR / 256;
  constexpr int KSTEP = 256 / CPR;  // key rows covered by one pass of 256 threads
  static_assert(LOADS >= 1, "tile loader");
  // two K/V tile buffers: tile j is computed from buffer j%2 while tile j+1's
  // registers land in the other one
  typedef uint16_t ktile_t[64 * KP];
  typedef uint16_t vtile_t[64 * VP];
  ktile_t* kl = reinterpret_cast<ktile_t*>(smem);
  vtile_t* vl = reinterpret_cast<vtile_t*>(smem + 2 * 64 * KP * 2);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const bool loader = NW == 4 || tid < 256;   // the threads that move tiles
  const Item it = load_item(item);
  // the item carries the sequence's first token and causal offset, and its
  // rows and key range are already clipped to the sequence
  const int t0 = it.t0;
  const int G = a.G;
  const int nrows = it.nrows;
  const int kv1 = min(it.kv1, a.MB * a.BS);

  const int rl = wave * 32 + n;
  const int r = it.row0 + rl;
  const bool row_ok = rl < nrows;
  const int tok = r / G;
  const int head = it.kvh * G + (r - tok * G);
  const int row_limit = a.causal ? tok + it.koff : INT_MAX;
  // an E4M3 cache holds K / k_scale and V / v_scale of each KV head: the
  // scores take k_scale inside the exponent's factor, O takes v_scale at the end
  const float sl2 = FP8 ? a.scale_log2 * ld_uniform(a.k_scale + it.kvh) : a.scale_log2;
  const float vsc = FP8 ? ld_uniform(a.v_scale + it.kvh) : 1.f;
  // every row of this wave sees keys up to at least wave_limit, and (with a
  // sliding window) no row of it sees a key below wave_lo
  const int wave_limit = a.causal ? (it.row0 + wave * 32) / G + it.koff : INT_MAX;
  const int wave_lo = a.window > 0 ? (it.row0 + wave * 32 + 31) / G + it.koff - (a.window - 1) : INT_MIN;
  const int row_lo = a.window > 0 ? tok + it.koff - (a.window - 1) : INT_MIN;
  // a wave skips the tiles that none of its rows sees (a wholly masked tile
  // adds nothing: the causal end of a block's last tile, and every tile of
  // the 8-wave items' second half-block past its rows), and a wave with no
  // rows skips all
  const bool wave_rows = wave * 32 < nrows;
  const int wave_last = a.causal ? (it.row0 + min(wave * 32 + 31, nrows - 1)) / G + it.koff : INT_MAX;

  bf16x8_t qf[NKT];
  if (row_ok) {
    const uint16_t* qp = a.q + ((int64_t)(t0 + tok) * a.H + head) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < NKT; ++t) qf[t] = ld16(qp + 16 * t);
  } else {
#pragma unroll
    for (int t = 0; t < NKT; ++t) qf[t] = zero8();
  }

  // loader: this thread moves chunk lcol of key rows lkey + KSTEP*i
  const int lkey = tid / CPR, lcol = tid % CPR;
  const int64_t row_elems = (int64_t)a.Hkv * D;
  const uint16_t* cbase = a.cache + (int64_t)it.kvh * D + lcol * 8;
  const int32_t* btrow = a.block_table + (int64_t)it.seq * a.bt_stride;
  const int bs_log2 = a.bs_log2;

  bf16x8_t kr[LOADS], vr[LOADS];
  // buffer-load geometry: bytes between key rows of one head, and this
  // thread's byte offset from the first key row of a pass (the same for
  // every pass and tile)
  const int row_bytes = (int)(row_elems * 2);
  const int ld_off = lkey * row_bytes + lcol * 16;
  const uint8_t* cache_b = reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)it.kvh * D * 2;
  auto load_tile = [&](int j0) {
    if constexpr (KSTEP <= 16) {
      // tiles start on a multiple of 16 and blocks hold a multiple of 16
      // keys, so the KSTEP keys of pass i share one block: the lookup is a
      // wave-uniform scalar load, and the pass is one bounds-checked buffer
      // load per plane through a resource that starts at the pass's first
      // key row and ends at the range's last key (rows past it read as
      // zero, with no per-lane branch or 64-bit address arithmetic)
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int kb = j0 + KSTEP * i;
        int nrec = 0;
        int64_t boff = 0;
        if (kb < kv1) {
          const int blk = (bs_log2 >= 0) ? (kb >> bs_log2) : (kb / a.BS);
          const int phys = ld_uniform(btrow + blk);
          if ((unsigned)phys < (unsigned)a.NB) {
            boff = ((int64_t)phys * a.BS + (kb - blk * a.BS)) * row_elems * 2;
            nrec = (min(KSTEP, kv1 - kb) - 1) * row_bytes + D * 2;
          }
        }
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(cache_b + boff), 0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(cache_b + a.plane * 2 + boff), 0, nrec, 0x00020000);
        kr[i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rk, ld_off, 0, 0));
        vr[i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rv, ld_off, 0, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int key = j0 + lkey + KSTEP * i;
        const int phys = (key < kv1) ? btrow[(bs_log2 >= 0) ? (key >> bs_log2) : (key / a.BS)] : -1;
        if ((unsigned)phys < (unsigned)a.NB) {
          int blk, off;
          if (bs_log2 >= 0) {
            blk = key >> bs_log2;
            off = key & (a.BS - 1);
          } else {
            blk = key / a.BS;
            off = key - blk * a.BS;
          }
          const uint16_t* p = cbase + ((int64_t)phys * a.BS + off) * row_elems;
          kr[i] = ld16(p);
          vr[i] = ld16(p + a.plane);
        } else {
          kr[i] = zero8();
          vr[i] = zero8();
        }
      }
    }
  };

  // Block-table entries of a tile's four 16-key groups (a tile starts on a
  // multiple of 16 keys and a block holds a multiple of 16, so each group
  // lies in one block): lane l loads the entry of group l % 4 with a vector
  // load one tile ahead.  Its wait is then counted in order with the K/V
  // loads and never holds LDS reads, as a scalar load's wait would.
  auto fetch_entries = [&](int j0) -> int {
    const int kg = min(j0 + 16 * (lane & 3), kv1 - 1);
    const int blk = (bs_log2 >= 0) ? (kg >> bs_log2) : (kg / a.BS);
    return btrow[blk];
  };
  auto load_tile_e = [&](int j0, int ent) {
    int ph[4], b16[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int kg = min(j0 + 16 * g, kv1 - 1);
      const int blk = (bs_log2 >= 0) ? (kg >> bs_log2) : (kg / a.BS);
      b16[g] = (j0 + 16 * g) - blk * a.BS;
      ph[g] = __builtin_amdgcn_readlane(ent, g);
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int kk = lkey + KSTEP * i;   // key within the tile
      int phys, bse;
      if constexpr (KSTEP <= 16) {       // pass i lies in one group
        phys = ph[(KSTEP * i) >> 4];
        bse = b16[(KSTEP * i) >> 4];
      } else {                           // two groups per pass: a bitwise
        // blend keeps the array indices constant (a select became a
        // dynamically indexed stack array)
        const int c = (KSTEP * i) >> 4;
        const int m = -((kk >> 4) & 1);
        phys = ph[c] ^ ((ph[c] ^ ph[c + 1]) & m);
        bse = b16[c] ^ ((b16[c] ^ b16[c + 1]) & m);
      }
      if (j0 + kk < kv1 && (unsigned)phys < (unsigned)a.NB) {
        const uint16_t* p = cbase + ((int64_t)phys * a.BS + bse + (kk & 15)) * row_elems;
        kr[i] = ld16(p);
        vr[i] = ld16(p + a.plane);
      } else {
        kr[i] = zero8();
        vr[i] = zero8();
      }
    }
  };

  // E4M3 cache: this thread moves 16-byte chunk lcol8 (16 elements) of key
  // rows lkey8 + KSTEP8*i of both planes and widens them to bf16 in LDS.  The
  // tile's four 16-key groups each lie in one cache block: four scalar
  // lookups, and each lane takes its group's.
  constexpr int CPR8 = D / 16;
  constexpr int LOADS8 = 64 * CPR8 / 256;
  constexpr int KSTEP8 = 256 / CPR8;
  static_assert(LOADS8 >= 1, "E4M3 tile loader");
  const int lkey8 = tid / CPR8, lcol8 = tid % CPR8;
  const uint8_t* cbase8 = reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)it.kvh * D + lcol8 * 16;
  u32x4_t k8[FP8 ? LOADS8 : 1], v8[FP8 ? LOADS8 : 1];
  auto load_tile8 = [&](int j0) {
    int phys16[4], base16[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int kg = min(j0 + 16 * g4, kv1 - 1);
      const int blk = (bs_log2 >= 0) ? (kg >> bs_log2) : (kg / a.BS);
      base16[g4] = (j0 + 16 * g4) - blk * a.BS;
      phys16[g4] = ld_uniform(btrow + blk);
    }
#pragma unroll
    for (int i = 0; i < LOADS8; ++i) {
      const int kk = KSTEP8 * i + lkey8;
      const int grp = kk >> 4;
      int ph = phys16[0], bs = base16[0];
#pragma unroll
      for (int g4 = 1; g4 < 4; ++g4) {
        ph = (grp == g4) ? phys16[g4] : ph;
        bs = (grp == g4) ? base16[g4] : bs;
      }
      if (j0 + kk < kv1 && (unsigned)ph < (unsigned)a.NB) {
        const uint8_t* p8 = cbase8 + ((int64_t)ph * a.BS + bs + (kk & 15)) * row_elems;
        k8[i] = *reinterpret_cast<const u32x4_t*>(p8);
        v8[i] = *reinterpret_cast<const u32x4_t*>(p8 + a.plane);
      } else {
        k8[i] = u32x4_t{0u, 0u, 0u, 0u};
        v8[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile8 = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS8; ++i) {
      const int kk = KSTEP8 * i + lkey8;
      u32x4_t lo, hi;
      e4m3x16_to_bf16(k8[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(kl[buf] + kk * KP + lcol8 * 16) = lo;
      *reinterpret_cast<u32x4_t*>(kl[buf] + kk * KP + lcol8 * 16 + 8) = hi;
      e4m3x16_to_bf16(v8[i], lo, hi);
      *reinterpret_cast<u32x4_t*>(vl[buf] + kk * VP + lcol8 * 16) = lo;
      *reinterpret_cast<u32x4_t*>(vl[buf] + kk * VP + lcol8 * 16 + 8) = hi;
    }
  };

  // l_run sums the fp32 probabilities (for the LSE), lr_run the bf16-rounded
  // ones that the PV product multiplies (for the normalisation of O)
  float m_run = kNegInf, l_run = 0.f, lr_run = 0.f;
  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  const int q16 = lane >> 4, s16 = lane & 15;
  const int koff = n * KP + 8 * h;
  const int voff = (4 * h + (s16 >> 2)) * VP + 16 * (q16 & 1) + 4 * (s16 & 3);

  auto tile = [&](int j0, int buf, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const uint16_t* kp0 = kl[buf] + koff;
    const uint16_t* vp0 = vl[buf] + voff;
    // S^T: two 32-key tiles; lane (n, h) reg i <- key j0 + 32u + 8(i/4) + 4h + i%4
    f32x16_t s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[u][i] = 0.f;
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kp0 + 32 * u * KP + 16 * t);
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[t], s[u], 0, 0, 0);
      }
    // raw scores; the scale (> 0) is applied inside the exponent, so the max
    // is taken on raw scores and scaled once
    float x[32];
    // the last visible key of this lane's row, relative to the lane's first
    // key j0 + 4h, so that each element compares a compile-time offset
    const int lim = min(kv1 - 1, row_limit) - j0 - 4 * h;
    // the first key of the row's sliding window, relative likewise
    const int lim_lo = (row_lo == INT_MIN) ? INT_MIN : row_lo - j0 - 4 * h;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[u][i];
        if constexpr (MASKED) {
          const int off = 32 * u + 8 * (i >> 2) + (i & 3);
          v = (off > lim || off < lim_lo) ? kNegInf : v;
        }
        x[16 * u + i] = v;
      }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, x[i]);
    mx = max_xor<32>(mx) * sl2;
    if (__builtin_expect(__any(mx > m_run + kRescaleSlack), 0)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};     // four independent partial sums
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl2, neg_m));
      ps[i & 3] += x[i];
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // P^T operands for the four 16-key steps: step ks = 2u + half uses
    // regs 8*half .. 8*half+7 of tile u
    bf16x8_t pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      pb[ks] = pack_bf16x8(x + 8 * ks);
      lr_run = add_bf16x8(pb[ks], lr_run);
    }
    // O^T += V^T P^T; A operand lane (m = d row, h) slots: keys kb+4h+0..3,
    // kb+8+4h+0..3 with kb = 16*ks, read transposed from LDS per 16-lane group
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint16_t* vr0 = vp0 + 16 * ks * VP;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8_t av = cat(lds_read_tr(vr0 + 32 * dt), lds_read_tr(vr0 + 8 * VP + 32 * dt));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], o[dt], 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int key = lkey + KSTEP * i;
      *reinterpret_cast<bf16x8_t*>(kl[buf] + key * KP + lcol * 8) = kr[i];
      *reinterpret_cast<bf16x8_t*>(vl[buf] + key * VP + lcol * 8) = vr[i];
    }
  };

  // one barrier per tile: after it, buffer buf holds tile j0 and every wave
  // has finished reading buffer buf^1 (tile j0-64), which the registers of
  // tile j0+64 overwrite once this tile's compute is done
  auto load_any = [&](int jt) {
    if constexpr (FP8)
      load_tile8(jt);
    else
      load_tile(jt);
  };
  auto store_any = [&](int b) {
    if constexpr (FP8)
      store_tile8(b);
    else
      store_tile(b);
  };
  int j0 = it.kv0, buf = 0;
  // bf16 cache at D = 64, where each lane would otherwise look up its own
  // key's block and wait for it: block entries of the next tile to load
  // (measured: 87 us against 93 us on 8 causal prefills of 256-2048 tokens;
  // at D = 128 the scalar lookups were as fast, at D = 256 the extra
  // register costs spills)
  constexpr bool VLOOKUP = !FP8 && D == 64;
  int ent = 0;
  if constexpr (!VLOOKUP) {
    if (loader && j0 < kv1) load_any(j0);
  } else if (loader) {
    if (j0 < kv1) load_tile_e(j0, fetch_entries(j0));
    if (j0 + 64 < kv1) ent = fetch_entries(j0 + 64);
  }
  // the first tile's loads and the Q loads are in flight together; all of
  // them must have landed before the loop: otherwise the wait-count pass
  // treats the Q loads as possibly in flight inside the loop and makes
  // every QK MFMA wait for the next tile's prefetch loads as well
  __builtin_amdgcn_s_waitcnt(0);
  if (loader && j0 < kv1) store_any(0);
  __syncthreads();
  for (; j0 < kv1; j0 += 64, buf ^= 1) {
    const bool more = j0 + 64 < kv1;
    if constexpr (!VLOOKUP) {
      if (more && loader) load_any(j0 + 64);
    } else if (more && loader) {
      load_tile_e(j0 + 64, ent);
      if (j0 + 128 < kv1) ent = fetch_entries(j0 + 128);
    }
    if (wave_rows && j0 <= wave_last) {
      if (j0 + 64 > kv1 || j0 + 63 > wave_limit || j0 < wave_lo)
        tile(j0, buf, Bool<true>{});
      else
        tile(j0, buf, Bool<false>{});
    }
    if (more && loader) store_any(buf ^ 1);
    __syncthreads();
  }

  l_run = sum_xor<32>(l_run);
  lr_run = sum_xor<32>(lr_run);
  if (!row_ok) return;
  float fo = 1.f;      // rescales O when a sink moves the reference
  if (a.s_aux && it.prow < 0) fo = add_sink(a.s_aux[head] * kLog2e, m_run, l_run, lr_run);
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : vsc * fo / lr_run;
  const float lse_v = empty ? kNegInf : (m_run + __log2f(l_run)) * kLn2;
  // lane (n, h) reg i of tile dt holds O^T[d = 32dt + 8(i/4) + 4h + i%4][row n]
  if (it.prow < 0) {
    const int64_t orow = (int64_t)(t0 + tok) * a.H + head;
    uint16_t* op = a.out + orow * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        uint2 w;
        w.x = pack_bf16x2(o[dt][4 * ig] * inv, o[dt][4 * ig + 1] * inv);
        w.y = pack_bf16x2(o[dt][4 * ig + 2] * inv, o[dt][4 * ig + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * dt + 8 * ig) = w;
      }
    if (h == 0 && a.lse) a.lse[orow] = lse_v;
  } else {
    float* pp = a.part_o + (int64_t)(it.prow + rl) * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        *reinterpret_cast<f32x4_t*>(pp + 32 * dt + 8 * ig) =
            f32x4_t{o[dt][4 * ig] * inv, o[dt][4 * ig + 1] * inv, o[dt][4 * ig + 2] * inv,
                    o[dt][4 * ig + 3] * inv};
    if (h == 0) a.part_lse[it.prow + rl] = lse_v;
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(256, (D >= 256 ? 1 : 2)) void attn_tiled_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[tiled_lds_bytes<D>()];
  tiled_body<D, FP8>(a, a.items + (int64_t)blockIdx.x * PA_ITEM_WORDS, smem);
}

// Tiled attention for items of up to 256 rows (launches with no small-row
// items, D <= 128): 8 waves of 32 rows share each K/V tile, so a tile is
// loaded and stored to LDS once per 256 rows instead of once per 128; one
// workgroup per compute unit holds the same 2 waves per SIMD as two
// 4-wave workgroups.
template <int D, bool FP8>
__global__ __launch_bounds__(512, 2) void attn_tiled_wide_kernel(AttnArgs a) {
  static_assert(D <= 128, "8 waves of a 256-row item fit the registers at D <= 128");
  __shared__ __attribute__((aligned(16))) uint8_t smem[tiled_lds_bytes<D>()];
  tiled_body<D, FP8, 8>(a, a.items + (int64_t)blockIdx.x * PA_ITEM_WORDS, smem);
}

// ---------------------------------------------------------------------------
// LDS-DMA tile loads (bf16 cache, D = 128, block size a power of two >= 16).
// K/V tiles go from HBM straight to LDS (buffer_load_dwordx4 ... lds): no
// register holds a tile in flight and no LDS store runs.
//   * A tile of kDmaTileKeys keys of one plane is kDmaTileKeys / 4 loads:
//     load i fills LDS bytes 1024 i .. 1024 i + 1023 with 8 key rows x 8
//     chunks of 16 bytes (8 whole 128-byte lines of the cache).  Lane l writes the 16 bytes at 16 l;
//     which chunk a lane fetches sets the layout, chosen so that the operand
//     reads hit all 64 banks once and their addresses are one register plus
//     constants:
//       K: unit 8 p + r8 holds row r8, chunk 8 ch + (p ^ (rg & 1))
//       V: unit 8 r8 + p holds row r8, chunk 8 ch + (p ^ 4 ((r8 >> 1) & 1))
//     (rg = i / 2, ch = i % 2).
//   * A 16-key group lies in one cache block (tiles start on a multiple of
//     16 keys), so one buffer resource per group covers it; keys past the
//     range and entries outside [0, NB) read as zeros.
//   * Block-table entries are scalar loads one tile ahead.
//   * The LDS address of each load passes through readfirstlane, so the
//     compiler ties no load to an LDS array and adds no wait of its own: the
//     explicit waits and barriers of the tile loop order loads and reads.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_void_ptr;
// keys per tile: 32-key tiles keep a workgroup at 32 KB of LDS and 160 VGPRs,
// so that three fit a compute unit (measured faster than 64-key tiles at two
// workgroups per compute unit on every prefill length tried)
constexpr int kDmaTileKeys = 32;
template <int N>
struct IntC {
  static constexpr int value = N;
};
// s_waitcnt with only the vector-memory count bounded (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Block-table entries of one tile's two 16-key groups, read by scalar
// loads: their waits count on lgkmcnt, which nothing else holds at the top
// of a tile iteration (the previous tile's LDS reads have all been
// consumed), so waiting for them never waits for a tile load in flight.
struct TileEntries {
  int e0, e1;
  __device__ int get(int g) const { return g == 0 ? e0 : e1; }
};
static_assert(kDmaTileKeys == 32, "TileEntries holds the entries of two 16-key groups");

// Stores one wave's 32 rows of O (lane (n, h) holds, in o[dt][4 ig + e],
// O^T[d = 32 dt + 8 ig + 4 h + e][row n], already normalised) through an
// 8 KB LDS region that no other wave touches: the 8-byte pieces go in with
// their 16-byte chunk index XORed by n mod 16, and come back 16 bytes per
// lane, 4 whole rows per instruction, so each wave issues 8 stores of whole
// 256-byte rows instead of 16 scattered 8-byte ones.  Rows at or past
// nrows_left are not stored.
template <int NDT>
__device__ __forceinline__ void store_rows_staged(const f32x16_t* o, float inv, uint8_t* stage,
                                                  int lane, uint16_t* out, int H, int t0,
                                                  int row0, int nrows_left, int G, int kvh) {
  constexpr int D = 32 * NDT;
  static_assert(D == 128, "16 chunks of 16 bytes per row");
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      uint2 w;
      w.x = pack_bf16x2(o[dt][4 * ig] * inv, o[dt][4 * ig + 1] * inv);
      w.y = pack_bf16x2(o[dt][4 * ig + 2] * inv, o[dt][4 * ig + 3] * inv);
      const int c = 4 * dt + ig;
      *reinterpret_cast<uint2*>(stage + n * 256 + ((c ^ (n & 15)) << 4) + 8 * h) = w;
    }
  const int c = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = 4 * i + (lane >> 4);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + lr * 256 + ((c ^ (lr & 15)) << 4));
    if (lr < nrows_left) {
      const int r = row0 + lr;
      const int tok = r / G;
      const int head = kvh * G + (r - tok * G);
      *reinterpret_cast<u32x4_t*>(out + ((int64_t)(t0 + tok) * H + head) * D + 8 * c) = v;
    }
  }
}


// ---------------------------------------------------------------------------
// 4-wave LDS-DMA tiled body (128-row items, bf16 cache, D = 128, block size a
// power of two >= 16): the DMA tile loads above, double-buffered (tile j+1
// loads while tile j is computed) in 32 KB, so that three workgroups fit a
// compute unit, beside each other or beside small-row items.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void tiled_dma4_body(const AttnArgs& a, const int32_t* item, uint8_t* kreg, uint8_t* vreg) {
  static_assert(D == 128, "4-wave LDS-DMA tiled body");
  // KT keys per tile: NG 16-key groups, NU 32-key halves of the score tile
  constexpr int KT = kDmaTileKeys, NKT = D / 16, NDT = D / 32, TILE = KT * 2 * D, NG = KT / 16,
                NU = KT / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const Item it = load_item(item);
  const int t0 = it.t0, G = a.G, nrows = it.nrows, kv0 = it.kv0;
  const int kv1 = min(it.kv1, a.MB * a.BS);
  const int nt = kv1 > kv0 ? (kv1 - kv0 + KT - 1) / KT : 0;
  const float sl2 = a.scale_log2;

  const int rl = wave * 32 + n;
  const int r = it.row0 + rl;
  const bool row_ok = rl < nrows;
  const int tok = r / G;
  const int head = it.kvh * G + (r - tok * G);
  const int row_limit = a.causal ? tok + it.koff : INT_MAX;
  const int row_lo = a.window > 0 ? tok + it.koff - (a.window - 1) : INT_MIN;
  const int wave_limit = a.causal ? (it.row0 + wave * 32) / G + it.koff : INT_MAX;
  const int wave_lo = a.window > 0 ? (it.row0 + wave * 32 + 31) / G + it.koff - (a.window - 1) : INT_MIN;
  const bool wave_rows = wave * 32 < nrows;
  const int wave_last = a.causal ? (it.row0 + min(wave * 32 + 31, nrows - 1)) / G + it.koff : INT_MAX;

  bf16x8_t qf[NKT];
  if (row_ok) {
    const uint16_t* qp = a.q + ((int64_t)(t0 + tok) * a.H + head) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < NKT; ++t) qf[t] = ld16(qp + 16 * t);
  } else {
#pragma unroll
    for (int t = 0; t < NKT; ++t) qf[t] = zero8();
  }

  // ---- loader (the DMA loads and layouts above): wave w (0..3) issues
  // i = w and w + 4 (16-key groups 0 and 1), with the same row within the
  // group (8 ((w / 2) & 1) + r8) and chunk for both
  const int64_t row_elems = (int64_t)a.Hkv * D;
  const int row_bytes = (int)(row_elems * 2);
  const int rgo = (wave >> 1) & 1, chh = wave & 1;
  const int voff_k = (8 * rgo + (lane & 7)) * row_bytes + ((8 * chh + ((lane >> 3) ^ rgo)) << 4);
  const int vr8 = lane >> 3;
  const int voff_v = (8 * rgo + vr8) * row_bytes + ((8 * chh + ((lane & 7) ^ (4 * ((vr8 >> 1) & 1)))) << 4);
  const uint8_t* cache_b = reinterpret_cast<const uint8_t*>(a.cache) + (int64_t)it.kvh * D * 2;
  const int32_t* btrow = a.block_table + (int64_t)it.seq * a.bt_stride;
  const int bs_log2 = a.bs_log2;
  const int last_blk = kv1 > 0 ? (kv1 - 1) >> bs_log2 : 0;
  const int64_t blk_bytes = (int64_t)row_bytes << bs_log2;
  const int64_t plane_bytes = a.plane * 2;

  // block-table entries of tile t's two 16-key groups (clamped to the
  // range's last block)
  auto fetch = [&](int t) -> TileEntries {
    const int k0 = kv0 + KT * t;
    return TileEntries{ld_uniform(btrow + min(k0 >> bs_log2, last_blk)),
                       ld_uniform(btrow + min((k0 + 16) >> bs_log2, last_blk))};
  };
  // the LDS address passes through readfirstlane, so that the compiler ties
  // no load to an LDS array and adds no wait of its own (the waits and
  // barriers of the loop order them); the small-row body shares lds_a
  auto dma = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* dst, int voff) {
    const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)dst);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(uintptr_t)la, 16, voff, 0, 0, 0);
  };
  auto load_tile = [&](int t, uint8_t* kd, uint8_t* vd, const TileEntries& ent) {
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int grp = q;
      const int g = wave + 4 * q;
      const int phys = ent.get(grp);
      const int key0 = kv0 + KT * t + 16 * grp;
      const bool ok = (key0 < kv1) & ((unsigned)phys < (unsigned)a.NB);
      const int64_t x = (int64_t)phys * blk_bytes + (int64_t)(key0 & (a.BS - 1)) * row_bytes;
      const int64_t boff = x & -(int64_t)ok;
      const int nrec = ((min(16, kv1 - key0) - 1) * row_bytes + D * 2) & -(int)ok;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(cache_b + boff), 0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(cache_b + plane_bytes + boff), 0, nrec, 0x00020000);
      dma(rk, kd + 1024 * g, voff_k);
      dma(rv, vd + 1024 * g, voff_v);
    }
  };

  // ---- read addresses.  K operand of k-step t, key half u (row r = n + 32u,
  // chunk C = 2t + h): 2048 (r / 8) + 1024 (C / 8) + 128 ((C % 8) ^ ((r / 8) & 1))
  // + 16 (r % 8) = kbase + 8192 u + 1024 (t / 4) + 256 (t % 4).  V operand of d
  // tile dt, 16-key step ks, second half e (row 16 ks + 8 e + r8, local chunk
  // cl of the tile's 4): vbase(dt % 2) + 4096 ks + 2048 e + 1024 (dt / 2).
  // Both are conflict-free: the 16 lanes of a K read and the 32 lanes of a
  // transposing read cover all 64 banks once.
  const int n8 = n >> 3;
  const int kbase = 2048 * n8 + 128 * (h ^ (n8 & 1)) + 16 * (n & 7);
  const int q16 = lane >> 4, s16 = lane & 15;
  const int r8v = 4 * h + (s16 >> 2);
  const int clv = 2 * (q16 & 1) + ((s16 & 3) >> 1);
  const int vbase0 = 128 * r8v + 16 * clv + 8 * (s16 & 1) + 64 * ((r8v >> 1) & 1);
  const int vbase1 = vbase0 ^ 64;

  float m_run = kNegInf, l_run = 0.f, lr_run = 0.f;
  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  // (forced inline: three unrolled calls exceed the inliner's budget, and an
  // outlined tile would keep O and the row state in scratch memory)
  auto tile = [&](int j0, const uint8_t* kb, const uint8_t* vb, bool masked) __attribute__((always_inline)) {
    f32x16_t s[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[u][i] = 0.f;
    constexpr int NR = NU * NKT, AHEAD = NR / 2;
    bf16x8_t kr[NR];
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        kr[NU * t + u] = *reinterpret_cast<const bf16x8_t*>(kb + kbase + 8192 * u + 1024 * (t >> 2) + 256 * (t & 3));
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[NU * t + u], qf[t], s[u], 0, 0, 0);
    // K operand reads run AHEAD of the matrix ops (left to itself the
    // scheduler kept one read in flight and waited for it before each
    // product): AHEAD reads, then one product and one read in turn
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);     // DS reads
#pragma unroll
    for (int i = 0; i < NR - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
    float x[16 * NU];
    const int lim = min(kv1 - 1, row_limit) - j0 - 4 * h;
    const int lim_lo = (row_lo == INT_MIN) ? INT_MIN : row_lo - j0 - 4 * h;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[16 * u + i] = s[u][i];
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16 * NU; ++i) {
        const int off = 32 * (i >> 4) + 8 * ((i & 15) >> 2) + (i & 3);
        x[i] = (off > lim || off < lim_lo) ? kNegInf : x[i];
      }
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 16 * NU; ++i) mx = fmaxf(mx, x[i]);
    mx = max_xor<32>(mx) * sl2;
    if (__builtin_expect(__any(mx > m_run + kRescaleSlack), 0)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16 * NU; ++i) {
      x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl2, neg_m));
      ps[i & 3] += x[i];
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    bf16x8_t pb[NG];
#pragma unroll
    for (int ks = 0; ks < NG; ++ks) {
      pb[ks] = pack_bf16x8(x + 8 * ks);
      lr_run = add_bf16x8(pb[ks], lr_run);
    }
#pragma unroll
    for (int ks = 0; ks < NG; ++ks) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint8_t* p0 = vb + ((dt & 1) ? vbase1 : vbase0) + 4096 * ks + 1024 * (dt >> 1);
        const bf16x8_t av = cat(lds_read_tr(reinterpret_cast<const uint16_t*>(p0)),
                                lds_read_tr(reinterpret_cast<const uint16_t*>(p0 + 2048)));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], o[dt], 0, 0, 0);
      }
    }
  };

  // ---- double buffer: iteration j issues tile j+1's loads into the other
  // slot after its barrier and computes tile j; the loop starts one tile
  // early (j = -1 only issues loads)
  TileEntries e_cur = nt > 0 ? fetch(0) : TileEntries{0, 0};   // entries of tile j+1 in iteration j
  TileEntries e_next = e_cur;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  auto iteration = [&](auto pc, int j) {
    constexpr int P = decltype(pc)::value & 1;    // slot of tile j
    // this wave's loads of tile j have landed; after the barrier so have
    // every wave's, and no wave reads tile j-1, whose slot tile j+1's loads
    // overwrite.  Loads stop at the last tile, so that the epilogue finds the
    // other slot empty.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("s_barrier" ::: "memory");
    if (j + 2 < nt) e_next = fetch(j + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < nt) load_tile(j + 1, kreg + TILE * (P ^ 1), vreg + TILE * (P ^ 1), e_cur);
    e_cur = e_next;
    const int j0 = kv0 + KT * j;
    if (j >= 0 && wave_rows && j0 <= wave_last)
      tile(j0, kreg + TILE * P, vreg + TILE * P, j0 + KT > kv1 || j0 + KT - 1 > wave_limit || j0 < wave_lo);
  };
  for (int j = nt > 0 ? -1 : 0;;) {
    if (j >= nt) break;
    iteration(IntC<1>{}, j++);
    if (j >= nt) break;
    iteration(IntC<0>{}, j++);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // ---- epilogue (as attn_tiled_kernel; whole outputs go through LDS)
  const float l = sum_xor<32>(l_run);
  float lr = sum_xor<32>(lr_run);
  float mr = m_run, ll = l, fo = 1.f;
  if (a.s_aux && it.prow < 0 && row_ok) fo = add_sink(a.s_aux[head] * kLog2e, mr, ll, lr);
  const bool empty = !(ll > 0.f);
  const float inv = empty ? 0.f : fo / lr;
  const float lse_v = empty ? kNegInf : (mr + __log2f(ll)) * kLn2;
  if (it.prow < 0) {
    // no load is in flight (loads stop at the last tile), and after this
    // barrier no wave reads a slot: both slots of both planes, 32 KB, 8 KB
    // per wave
    asm volatile("s_barrier" ::: "memory");
    uint8_t* region = (wave < 2 ? kreg : vreg) + 8192 * (wave & 1);
    store_rows_staged<NDT>(o, inv, region, lane, a.out, a.H, t0, it.row0 + wave * 32,
                           nrows - wave * 32, G, it.kvh);
    if (h == 0 && a.lse && row_ok) a.lse[(int64_t)(t0 + tok) * a.H + head] = lse_v;
  } else {
    if (!row_ok) return;
    float* pp = a.part_o + (int64_t)(it.prow + rl) * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig)
        *reinterpret_cast<f32x4_t*>(pp + 32 * dt + 8 * ig) =
            f32x4_t{o[dt][4 * ig] * inv, o[dt][4 * ig + 1] * inv, o[dt][4 * ig + 2] * inv,
                    o[dt][4 * ig + 3] * inv};
    if (h == 0) a.part_lse[it.prow + rl] = lse_v;
  }
}

// 128-row tiled items alone (bf16 cache, D = 128, power-of-two block size):
// three 4-wave workgroups per compute unit, each double-buffering its tiles,
// so that one workgroup's first loads and last stores overlap the others'
// tiles.  It measured faster than an 8-wave form with 256-row items sharing
// each tile, at every length tried (592-1811 and 8192 tokens).
template <int D>
__global__ __launch_bounds__(256, 3) void attn_tiled_dma4_kernel(AttnArgs a) {
  constexpr int TILE = kDmaTileKeys * 2 * D;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b[2 * TILE];
  tiled_dma4_body<D>(a, a.items + (int64_t)blockIdx.x * PA_ITEM_WORDS, lds_a, lds_b);
}

// Mixed launch of a bf16 cache at D = 128 with a power-of-two block size:
// small-row items as in attn_small_kernel (two load steps in flight), tiled
// items by the 4-wave LDS-DMA body, three workgroups per compute unit.  The
// small body's staging area and the K slots share lds_a.
template <int D>
__global__ __launch_bounds__(256, 3) void attn_mixed_dma_kernel(AttnArgs a) {
  constexpr int TILE = kDmaTileKeys * 2 * D;
  constexpr int LA = small_lds_bytes<D>() > 2 * TILE ? small_lds_bytes<D>() : 2 * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a[(LA + 1023) / 1024 * 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b[2 * TILE];
  const int32_t* item = a.items + (int64_t)blockIdx.x * PA_ITEM_WORDS;
  if (ld_uniform(item + 7))
    tiled_dma4_body<D>(a, item, lds_a, lds_b);
  else
    small_body<D, false, SmallCfg<D>::PF_SMALL>(a, item, lds_a);
}

// ---------------------------------------------------------------------------
// Mixed launch: when a batch has both decode-like and prefill rows, one grid
// runs both kinds of item (word 7 of an item: 0 small-row, 1 tiled), in the
// planner's longest-first order, so the HBM-bound small-row workgroups and
// the matrix-core-bound tiled ones share the compute units instead of
// running one kernel after the other.
// ---------------------------------------------------------------------------
template <int D, bool FP8>
__global__ __launch_bounds__(256, (D >= 256 ? 1 : 2)) void attn_mixed_kernel(AttnArgs a) {
  constexpr int L = small_lds_bytes<D>() > tiled_lds_bytes<D>() ? small_lds_bytes<D>() : tiled_lds_bytes<D>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[L];
  const int32_t* item = a.items + (int64_t)blockIdx.x * PA_ITEM_WORDS;
  if (ld_uniform(item + 7))
    tiled_body<D, FP8>(a, item, smem);
  else
    small_body<D, FP8, SmallCfg<D>::PF>(a, item, smem);
}

// ---------------------------------------------------------------------------
// Split-KV reduction: one workgroup per (reduce item, row); its 4 waves take
// every 4th split, each lane D/64 elements of the row.  Partials hold O
// normalised by its own row sum and the natural-log lse of that split; a
// wave merges its splits online (running max, rescaled sum), loading a
// split's lse and O together, and the 4 waves' states meet in LDS.  The item
// carries the sequence's first token and its rows are all valid (the
// planner clips them), so the only loads on the way are the partials.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void split_reduce_kernel(
    const int32_t* __restrict__ ritems, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, uint16_t* __restrict__ out, float* __restrict__ lse, int H,
    int G, const float* __restrict__ s_aux) {
  constexpr int EPL = D / 64;
  static_assert(EPL >= 1, "split reduce");
  __shared__ float s_m[4], s_l[4];
  __shared__ __attribute__((aligned(16))) float s_o[4][D];
  const int32_t* p = ritems + (int64_t)blockIdx.x * PA_ITEM_WORDS;
  const int kvh = ld_uniform(p + 1), row0 = ld_uniform(p + 2);
  const int prow_n = ld_uniform(p + 3), prow0 = ld_uniform(p + 4), nsplit = ld_uniform(p + 5);
  const int t0 = ld_uniform(p + 6);
  const int row = blockIdx.y;
  if (row >= prow_n) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // online merge over this wave's splits, in the log2 domain
  float m = kNegInf, L = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int s = wave; s < nsplit; s += 4) {
    const int pr = prow0 + s * prow_n + row;
    const float ls = part_lse[pr] * kLog2e;
    float v[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = part_o[(int64_t)pr * D + lane * EPL + e];
    const float m_new = fmaxf(m, ls);
    if (m_new == kNegInf) continue;   // nothing seen yet: both sides empty
    const float a = __builtin_amdgcn_exp2f(m - m_new);   // 0 when m = -inf
    const float b = __builtin_amdgcn_exp2f(ls - m_new);  // 0 when ls = -inf
    L = L * a + b;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * a + b * v[e];
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_o[wave][lane * EPL + e] = acc[e];
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = L;
  }
  __syncthreads();
  if (wave != 0) return;
  const int rr = row0 + row;
  const int tok = rr / G;
  const int head = kvh * G + (rr - tok * G);
  float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float w[4], Lt = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[k] = (s_m[k] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(s_m[k] - M);
    Lt += w[k] * s_l[k];
  }
  // a sink joins the merged denominator once (the partials exclude it)
  float fo = 1.f;
  if (s_aux) {
    float unused = 0.f;
    fo = add_sink(ld_uniform(s_aux + head) * kLog2e, M, Lt, unused);
  }
  const bool empty = !(Lt > 0.f);
  const float inv = empty ? 0.f : fo / Lt;
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    acc[e] = ((w[0] * s_o[0][lane * EPL + e] + w[1] * s_o[1][lane * EPL + e]) +
              (w[2] * s_o[2][lane * EPL + e] + w[3] * s_o[3][lane * EPL + e])) * inv;
  const int64_t orow = (int64_t)(t0 + tok) * H + head;
  uint16_t* op = out + orow * D + lane * EPL;
  if constexpr (EPL == 1) {
    op[0] = (uint16_t)(pack_bf16x2(acc[0], 0.f) & 0xffffu);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; e += 2)
      *reinterpret_cast<uint32_t*>(op + e) = pack_bf16x2(acc[e], acc[e + 1]);
  }
  if (lane == 0 && lse) lse[orow] = empty ? kNegInf : (M + __log2f(Lt)) * kLn2;
}

// ---------------------------------------------------------------------------
// Two-way merge of (out, lse) partial states.  A row of D elements is
// cpr = D/8 chunks of 8; a wave holds 64 >> p2 rows of 1 << p2 lanes (the
// smallest power of two >= cpr, cpr <= 64), so a lane's row and chunk come
// from shifts.  out may alias po or so: each lane reads its 8 elements before
// writing them.  out_lse does not alias pl or sl (the entry point checks).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_states_kernel(
    uint16_t* out, float* __restrict__ out_lse, const uint16_t* po, const float* __restrict__ pl,
    const uint16_t* so, const float* __restrict__ sl, int64_t rows, int32_t cpr, int32_t p2) {
  const int lane = threadIdx.x & 63;
  const int c = lane & ((1 << p2) - 1);
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 >> p2) + (lane >> p2);
  if (row >= rows || c >= cpr) return;
  const float lp = pl[row], ls = sl[row];
  const float M = fmaxf(lp, ls);
  const int64_t off = row * cpr * 8 + c * 8;
  const uint4 wp = *reinterpret_cast<const uint4*>(po + off);
  const uint4 ws = *reinterpret_cast<const uint4*>(so + off);
  float res[8];
  float lse_v;
  if (M == kNegInf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = 0.f;
    lse_v = kNegInf;
  } else {
    const float wa = (lp == kNegInf) ? 0.f : expf(lp - M);
    const float wb = (ls == kNegInf) ? 0.f : expf(ls - M);
    const float den = wa + wb;
    const float ia = wa / den, ib = wb / den;
    const uint32_t pw[4] = {wp.x, wp.y, wp.z, wp.w};
    const uint32_t sw[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      res[2 * e] = ia * __uint_as_float(pw[e] << 16) + ib * __uint_as_float(sw[e] << 16);
      res[2 * e + 1] = ia * __uint_as_float(pw[e] & 0xffff0000u) +
                       ib * __uint_as_float(sw[e] & 0xffff0000u);
    }
    lse_v = M + logf(den);
  }
  *reinterpret_cast<bf16x8_t*>(out + off) = pack_bf16x8(res);
  if (c == 0 && out_lse) out_lse[row] = lse_v;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int D, bool FP8>
pa_status launch_fwd(const AttnArgs& base, const pa_plan_info* plan, const int32_t* worklist,
                     hipStream_t stream) {
  const int32_t* items = worklist + PA_WORKLIST_HEADER_WORDS;
  AttnArgs a = base;
  a.items = items;
  if (plan->num_small_items > 0 && plan->num_tiled_items > 0) {
    bool launched = false;
    if constexpr (D == 128 && !FP8) {
      if (a.bs_log2 >= 4) {
        hipLaunchKernelGGL((attn_mixed_dma_kernel<D>),
                           dim3(plan->num_small_items + plan->num_tiled_items), dim3(256), 0, stream, a);
        launched = true;
      }
    }
    if (!launched)
      hipLaunchKernelGGL((attn_mixed_kernel<D, FP8>),
                         dim3(plan->num_small_items + plan->num_tiled_items), dim3(256), 0, stream, a);
  } else if (plan->num_small_items > 0) {
    hipLaunchKernelGGL((attn_small_kernel<D, FP8>), dim3(plan->num_small_items), dim3(256), 0, stream, a);
  } else if (plan->num_tiled_items > 0) {
    bool launched = false;
    if constexpr (D <= 128) {
      if (plan->tiled_rows == PA_TILED_ROWS_WIDE) {
        hipLaunchKernelGGL((attn_tiled_wide_kernel<D, FP8>), dim3(plan->num_tiled_items),
                           dim3(512), 0, stream, a);
        launched = true;
      }
    }
    if constexpr (D == 128 && !FP8) {
      if (!launched && a.bs_log2 >= 4) {
        hipLaunchKernelGGL((attn_tiled_dma4_kernel<D>), dim3(plan->num_tiled_items), dim3(256), 0,
                           stream, a);
        launched = true;
      }
    }
    if (!launched)
      hipLaunchKernelGGL((attn_tiled_kernel<D, FP8>), dim3(plan->num_tiled_items), dim3(256), 0,
                         stream, a);
  }
  if (plan->num_reduce_items > 0) {
    const int32_t* r =
        items + (int64_t)(plan->num_small_items + plan->num_tiled_items) * PA_ITEM_WORDS;
    hipLaunchKernelGGL(split_reduce_kernel<D>, dim3(plan->num_reduce_items, plan->max_reduce_rows),
                       dim3(256), 0, stream,
                       r, base.part_o, base.part_lse, base.out, base.lse, base.H, base.G,
                       base.s_aux);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

pa_status pa_upload_words(const int32_t* host_src, int32_t* dev_dst, int64_t n_words,
                          hipStream_t stream) {
  if (n_words < 0 || n_words > ((int64_t)1 << 34)) return PA_ERR_INVALID_ARGUMENT;
  if (n_words == 0) return PA_OK;
  if (!host_src || !dev_dst || !aligned(host_src, 16) || !aligned(dev_dst, 16))
    return PA_ERR_INVALID_ARGUMENT;
  // the device's address of the pinned buffer; fails for memory the device
  // cannot read, which is then an error instead of a fault
  void* src_dev = nullptr;
  if (hipHostGetDevicePointer(&src_dev, const_cast<int32_t*>(host_src), 0) != hipSuccess ||
      !src_dev) {
    (void)hipGetLastError();
    return PA_ERR_INVALID_ARGUMENT;
  }
  const int64_t n16 = (n_words + 3) / 4;
  const uint32_t blocks = (uint32_t)((n16 + 255) / 256);
  hipLaunchKernelGGL(upload_words_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const int32_t*>(src_dev), dev_dst, n_words);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_reshape_and_cache(const void* key, const void* value, int64_t key_row_stride,
                               int64_t value_row_stride, void* kv_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_size, int32_t num_blocks,
                               int32_t block_size, hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || head_size % 8 != 0 ||
      head_size > 4096 || num_blocks <= 0 || block_size <= 0 || block_size % 16 != 0)
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_row_stride < row || value_row_stride < row || key_row_stride % 8 != 0 ||
      value_row_stride % 8 != 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !kv_cache || !slot_mapping) return PA_ERR_INVALID_ARGUMENT;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(kv_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t plane = (int64_t)num_blocks * block_size * row;
  const int32_t cpr = (int32_t)(row / 8);
  const int32_t per_block = 4 * RC_TOKENS_PER_WAVE;
  const uint32_t blocks = (uint32_t)((num_tokens + per_block - 1) / per_block);
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                     key_row_stride, value_row_stride, static_cast<uint16_t*>(kv_cache),
                     slot_mapping, num_tokens, cpr, row, plane, (int64_t)num_blocks * block_size);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t key_row_stride,
                                   int64_t value_row_stride, void* kv_cache,
                                   const int64_t* slot_mapping, const float* k_scale,
                                   const float* v_scale, int32_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_size, int32_t num_blocks, int32_t block_size,
                                   hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_size <= 0 || head_size % 16 != 0 ||
      head_size > 4096 || num_blocks <= 0 || block_size <= 0 || block_size % 16 != 0)
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t row = (int64_t)num_kv_heads * head_size;
  if (key_row_stride < row || value_row_stride < row || key_row_stride % 8 != 0 ||
      value_row_stride % 8 != 0)
    return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !kv_cache || !slot_mapping || !k_scale || !v_scale)
    return PA_ERR_INVALID_ARGUMENT;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(kv_cache, 16) ||
      !aligned(slot_mapping, 8) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t plane = (int64_t)num_blocks * block_size * row;   // bytes
  const int32_t cpr = (int32_t)(row / 16);
  const uint32_t blocks = (uint32_t)((num_tokens + 3) / 4);
  hipLaunchKernelGGL(reshape_and_cache_fp8_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                     key_row_stride, value_row_stride, static_cast<uint8_t*>(kv_cache),
                     slot_mapping, k_scale, v_scale, num_tokens, cpr, head_size / 16, row, plane,
                     (int64_t)num_blocks * block_size);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"

namespace {

// The split-KV partials of pa_varlen_fwd_noalloc: a device array compiled
// into the library (each GPU holds its own copy until the process ends).
// Host code never passes `scratch` itself to a kernel (on the host it names
// a stand-in, not the device address): the address is resolved once per
// device with hipGetSymbolAddress, with that device current, and kept.
static __device__ __attribute__((aligned(256))) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

// pa_varlen_fwd, pa_varlen_fwd_fp8, pa_varlen_fwd_ex and
// pa_varlen_fwd_noalloc: fp8 selects the E4M3 cache with its per-KV-head
// scales; use_scratch puts the partials in `scratch` instead of `workspace`
pa_status varlen_fwd(const pa_attn_params* p, const pa_plan_info* plan, const int32_t* worklist,
                     const void* q, const void* kv_cache, const int32_t* cu_seqlens_q,
                     const int32_t* seqused_k, const int32_t* block_table, const float* k_scale,
                     const float* v_scale, bool fp8, const float* s_aux, int32_t num_tokens,
                     void* out, float* lse, void* workspace, size_t workspace_bytes,
                     bool use_scratch, hipStream_t stream) {
  pa_status st = pa::check_params(p);
  if (st != PA_OK) return st;
  if (!plan) return PA_ERR_INVALID_ARGUMENT;
  if (plan->batch != p->batch || plan->num_heads != p->num_heads ||
      plan->num_kv_heads != p->num_kv_heads || plan->head_size != p->head_size ||
      plan->causal != p->causal || plan->num_tokens != num_tokens ||
      plan->sliding_window != p->sliding_window)
    return PA_ERR_INVALID_ARGUMENT;
  if (plan->num_small_items < 0 || plan->num_tiled_items < 0 || plan->num_reduce_items < 0 ||
      plan->num_partial_rows < 0 || plan->max_reduce_rows < 0 ||
      plan->max_reduce_rows > plan->tiled_rows ||
      (plan->num_reduce_items > 0 && plan->max_reduce_rows == 0))
    return PA_ERR_INVALID_ARGUMENT;
  // wide tiled blocks only in launches of tiled items alone, at D <= 128
  if (plan->tiled_rows != PA_TILED_ROWS &&
      (plan->tiled_rows != PA_TILED_ROWS_WIDE || plan->num_small_items > 0 || p->head_size > 128))
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t n_items =
      (int64_t)plan->num_small_items + plan->num_tiled_items + plan->num_reduce_items;
  if (plan->worklist_bytes != (size_t)(PA_WORKLIST_HEADER_WORDS + n_items * PA_ITEM_WORDS) * 4)
    return PA_ERR_INVALID_ARGUMENT;
  if (use_scratch) {
    if (plan->workspace_bytes > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE_TOO_SMALL;
  } else {
    if (workspace_bytes < plan->workspace_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    if (plan->workspace_bytes > 0 && (!workspace || !aligned(workspace, 256)))
      return PA_ERR_INVALID_ARGUMENT;
  }
  if (n_items == 0) return PA_OK;
  if (!worklist || !q || !kv_cache || !cu_seqlens_q || !seqused_k || !block_table || !out)
    return PA_ERR_INVALID_ARGUMENT;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return PA_ERR_INVALID_ARGUMENT;
  if (s_aux && !aligned(s_aux, 4)) return PA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(worklist, 4) ||
      (lse && !aligned(lse, 4)))
    return PA_ERR_INVALID_ARGUMENT;
  if (plan->num_small_items > 0 && p->num_heads / p->num_kv_heads > PA_SMALL_MAX_ROWS)
    return PA_ERR_INVALID_ARGUMENT;
  // every check has passed: only now the first call on a device resolves
  // its scratch address (no partial row needs clearing: each one is written
  // before the reduce of the same call reads it)
  if (use_scratch) {
    workspace = nullptr;
    if (plan->workspace_bytes > 0) {
      st = scratch_address(&workspace);
      if (st != PA_OK) return st;
    }
  }
  AttnArgs a;
  a.items = nullptr;
  a.q = static_cast<const uint16_t*>(q);
  a.cache = static_cast<const uint16_t*>(kv_cache);
  a.cu = cu_seqlens_q;
  a.seqused_k = seqused_k;
  a.block_table = block_table;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const size_t o_bytes = (size_t)plan->num_partial_rows * p->head_size * sizeof(float);
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                    (o_bytes + 255) / 256 * 256)
                         : nullptr;
  a.plane = (int64_t)p->num_blocks * p->block_size * p->num_kv_heads * p->head_size;
  a.NB = p->num_blocks;
  a.H = p->num_heads;
  a.Hkv = p->num_kv_heads;
  a.G = p->num_heads / p->num_kv_heads;
  a.BS = p->block_size;
  a.MB = p->max_blocks_per_seq;
  a.bt_stride = p->block_table_stride ? p->block_table_stride : p->max_blocks_per_seq;
  a.causal = p->causal;
  a.bs_log2 = -1;
  for (int b = 0; b < 31; ++b)
    if ((1 << b) == p->block_size) a.bs_log2 = b;
  a.scale_log2 = p->scale * kLog2e;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.s_aux = s_aux;
  a.window = p->sliding_window;
  switch (p->head_size) {
    case 64: return fp8 ? launch_fwd<64, true>(a, plan, worklist, stream)
                        : launch_fwd<64, false>(a, plan, worklist, stream);
    case 128: return fp8 ? launch_fwd<128, true>(a, plan, worklist, stream)
                         : launch_fwd<128, false>(a, plan, worklist, stream);
    case 256: return fp8 ? launch_fwd<256, true>(a, plan, worklist, stream)
                         : launch_fwd<256, false>(a, plan, worklist, stream);
  }
  return PA_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

pa_status pa_varlen_fwd(const pa_attn_params* p, const pa_plan_info* plan, const int32_t* worklist,
                        const void* q, const void* kv_cache, const int32_t* cu_seqlens_q,
                        const int32_t* seqused_k, const int32_t* block_table, int32_t num_tokens,
                        void* out, float* lse, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return varlen_fwd(p, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table, nullptr,
                    nullptr, false, nullptr, num_tokens, out, lse, workspace, workspace_bytes,
                    false, stream);
}

pa_status pa_varlen_fwd_ex(const pa_attn_params* p, const pa_plan_info* plan,
                           const int32_t* worklist, const void* q, const void* kv_cache,
                           const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                           const int32_t* block_table, const pa_fwd_options* opt,
                           int32_t num_tokens, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (!opt || (opt->kv_dtype != PA_KV_BF16 && opt->kv_dtype != PA_KV_E4M3))
    return PA_ERR_INVALID_ARGUMENT;
  return varlen_fwd(p, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table,
                    opt->k_scale, opt->v_scale, opt->kv_dtype == PA_KV_E4M3, opt->s_aux,
                    num_tokens, out, lse, workspace, workspace_bytes, false, stream);
}

pa_status pa_varlen_fwd_noalloc(const pa_attn_params* p, const pa_plan_info* plan,
                                const int32_t* worklist, const void* q, const void* kv_cache,
                                const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                const int32_t* block_table, const pa_fwd_options* opt,
                                int32_t num_tokens, void* out, float* lse, hipStream_t stream) {
  if (opt && opt->kv_dtype != PA_KV_BF16 && opt->kv_dtype != PA_KV_E4M3)
    return PA_ERR_INVALID_ARGUMENT;
  const bool fp8 = opt && opt->kv_dtype == PA_KV_E4M3;
  return varlen_fwd(p, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table,
                    opt ? opt->k_scale : nullptr, opt ? opt->v_scale : nullptr, fp8,
                    opt ? opt->s_aux : nullptr, num_tokens, out, lse, nullptr, 0, true, stream);
}

pa_status pa_varlen_fwd_fp8(const pa_attn_params* p, const pa_plan_info* plan,
                            const int32_t* worklist, const void* q, const void* kv_cache,
                            const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                            const int32_t* block_table, const float* k_scale, const float* v_scale,
                            int32_t num_tokens, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return varlen_fwd(p, plan, worklist, q, kv_cache, cu_seqlens_q, seqused_k, block_table, k_scale,
                    v_scale, true, nullptr, num_tokens, out, lse, workspace, workspace_bytes,
                    false, stream);
}

pa_status pa_merge_attn_states(void* out, float* out_lse, const void* prefix_out,
                               const float* prefix_lse, const void* suffix_out,
                               const float* suffix_lse, int32_t num_tokens, int32_t num_heads,
                               int32_t head_size, hipStream_t stream) {
  if (num_tokens < 0 || num_heads <= 0 || head_size <= 0 || head_size % 8 != 0 || head_size > 512)
    return PA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PA_OK;
  if (!out || !prefix_out || !prefix_lse || !suffix_out || !suffix_lse)
    return PA_ERR_INVALID_ARGUMENT;
  if (!aligned(out, 16) || !aligned(prefix_out, 16) || !aligned(suffix_out, 16))
    return PA_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)num_tokens * num_heads;
  // out_lse must not overlap either input lse (the lanes of one row read the
  // inputs and one of them writes out_lse, in no fixed order)
  if (out_lse) {
    auto overlaps = [rows](const float* x, const float* y) { return x < y + rows && y < x + rows; };
    if (overlaps(out_lse, prefix_lse) || overlaps(out_lse, suffix_lse)) return PA_ERR_INVALID_ARGUMENT;
  }
  const int32_t cpr = head_size / 8;
  int32_t p2 = 0;
  while ((1 << p2) < cpr) ++p2;
  const int64_t rows_per_block = 4 * (64 >> p2);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks > INT32_MAX) return PA_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(merge_states_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<uint16_t*>(out), out_lse, static_cast<const uint16_t*>(prefix_out),
                     prefix_lse, static_cast<const uint16_t*>(suffix_out), suffix_lse, rows, cpr, p2);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
