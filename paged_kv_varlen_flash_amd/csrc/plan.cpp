// Host-side planner and argument checks for libpagedattn.
//
// The planner turns the host mirrors of cu_seqlens_q / seqused_k into a fixed
// work list, the ahead-of-time schedule of "FlashAttention 在 vLLM 中的实现分析"
// (section 7): which rows of which (sequence, KV head) each workgroup takes,
// which key range, and where split-KV partials go.  Pure host code: no HIP
// call is made here, so every check can run on a machine without a GPU.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "pagedattn.h"
#include "plan_internal.h"

namespace pa {

bool head_size_supported(int32_t d) {
  for (int i = 0; i < PA_NUM_HEAD_SIZES; ++i)
    if (pa_supported_head_sizes[i] == d) return true;
  return false;
}

pa_status check_params(const pa_attn_params* p) {
  if (!p) return PA_ERR_INVALID_ARGUMENT;
  if (p->batch < 0 || p->num_heads <= 0 || p->num_kv_heads <= 0) return PA_ERR_INVALID_ARGUMENT;
  if (p->num_heads % p->num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
  // the FlashAttention backend asks for a head size that is a multiple of 8
  // and at most 256 ("AttentionBackend" page, 境界と失敗)
  if (p->head_size <= 0 || p->head_size % 8 != 0 || p->head_size > 256)
    return PA_ERR_INVALID_ARGUMENT;
  if (!head_size_supported(p->head_size)) return PA_ERR_UNSUPPORTED;
  // block size must be a multiple of 16 (same page, and the FlashAttention
  // page's get_kv_cache_shape raises on any other size)
  if (p->block_size <= 0 || p->block_size % 16 != 0) return PA_ERR_INVALID_ARGUMENT;
  if (p->num_blocks <= 0 || p->max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARGUMENT;
  if (p->block_table_stride != 0 && p->block_table_stride < p->max_blocks_per_seq)
    return PA_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->max_blocks_per_seq * p->block_size > INT32_MAX / 2) return PA_ERR_INVALID_ARGUMENT;
  if (p->causal != 0 && p->causal != 1) return PA_ERR_INVALID_ARGUMENT;
  if (p->kv_cache_fp8 != 0 && p->kv_cache_fp8 != 1) return PA_ERR_INVALID_ARGUMENT;
  if (p->num_cus < 0 || p->num_cus > 65536) return PA_ERR_INVALID_ARGUMENT;
  // a sliding window is the causal band of its last W keys
  if (p->sliding_window < 0 || (p->sliding_window > 0 && !p->causal)) return PA_ERR_INVALID_ARGUMENT;
  // a softmax scale is positive (the kernels take row maxima on unscaled scores)
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return PA_ERR_INVALID_ARGUMENT;
  // byte offsets into the cache must fit in 64 bits with room to spare, and
  // every per-launch index the kernels form in 32 bits must fit
  const int64_t plane = (int64_t)p->num_blocks * p->block_size * p->num_kv_heads * p->head_size;
  if (plane <= 0 || plane > ((int64_t)1 << 40)) return PA_ERR_INVALID_ARGUMENT;
  return PA_OK;
}

namespace {

struct Unit {        // one (sequence, kv head, row block) with its visible key range
  int32_t seq, kvh, row0, nrows, kv_end;
  bool small;
  int32_t kv_begin;  // first key any row of the block sees (a multiple of 16)
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int32_t ceil_div32(int32_t a, int32_t b) { return (int32_t)(((uint32_t)a + (uint32_t)b - 1u) / (uint32_t)b); }

struct Item {        // one work item and its cost (keys x rows)
  int32_t w[PA_ITEM_WORDS];
  int64_t cost;
};

// Indices of `items` in order of decreasing cost, ties in list order: a
// least-significant-digit radix sort, one stable 256-bucket counting pass per
// byte of the largest cost, over packed 64-bit values ((largest cost - cost)
// above a 24-bit list index; costs are below 2^40: keys < 2^30, rows <= 128).
// The planner runs once per step on the host, and a comparison sort of a few
// thousand items took most of its time (chunked_prefill_mix: 228 us of
// planning per step before, 80-90 us after).
void order_by_cost(const std::vector<Item>& items, std::vector<uint32_t>& order) {
  const size_t n = items.size();
  order.resize(n);
  constexpr int kIdxBits = 24;
  int64_t maxc = 0;
  for (const Item& it : items) maxc = std::max(maxc, it.cost);
  if (n >= ((size_t)1 << kIdxBits) || maxc >= ((int64_t)1 << 40)) {
    for (size_t i = 0; i < n; ++i) order[i] = (uint32_t)i;
    std::stable_sort(order.begin(), order.end(),
                     [&](uint32_t a, uint32_t b) { return items[a].cost > items[b].cost; });
    return;
  }
  thread_local std::vector<uint64_t> va, vb;
  va.resize(n);
  vb.resize(n);
  for (size_t i = 0; i < n; ++i) va[i] = ((uint64_t)(maxc - items[i].cost) << kIdxBits) | i;
  if (n < 2048) {
    // a comparison sort of the same keys (same order) was faster below a
    // couple of thousand items (hipcc -O3): 25 us against 29 us for the
    // whole plan of 64 decode sequences; at 2160 items radix took 23 us
    // against 84 us
    std::sort(va.begin(), va.end());
    for (size_t i = 0; i < n; ++i) order[i] = (uint32_t)(va[i] & (((uint64_t)1 << kIdxBits) - 1));
    return;
  }
  uint64_t* src = va.data();
  uint64_t* dst = vb.data();
  for (int shift = kIdxBits; shift < 64 && (maxc >> (shift - kIdxBits)) > 0; shift += 8) {
    size_t count[257] = {};
    for (size_t i = 0; i < n; ++i) ++count[(src[i] >> shift & 255) + 1];
    for (int d = 0; d < 256; ++d) count[d + 1] += count[d];
    for (size_t i = 0; i < n; ++i) dst[count[src[i] >> shift & 255]++] = src[i];
    std::swap(src, dst);
  }
  for (size_t i = 0; i < n; ++i) order[i] = (uint32_t)(src[i] & (((uint64_t)1 << kIdxBits) - 1));
}

// Writes items in order of decreasing cost, ties in list order, and returns
// the end of what it wrote.
int32_t* emit_by_cost(const std::vector<Item>& items, int32_t* dst) {
  thread_local std::vector<uint32_t> order;
  order_by_cost(items, order);
  for (uint32_t i : order) {
    std::memcpy(dst, items[i].w, sizeof(Item::w));
    dst += PA_ITEM_WORDS;
  }
  return dst;
}

// Items of one kind as a longest-first queue, and the proportional merge of
// a small-row and a tiled queue: the kind further behind its share goes
// next, so that HBM-bound small-row workgroups and matrix-core-bound tiled
// ones share the compute units throughout the launch.
void merge_proportional(const std::vector<const Item*>& qs, const std::vector<const Item*>& qt,
                        std::vector<const Item*>& out) {
  const uint64_t ns = qs.size(), nt = qt.size();
  uint64_t is = 0, itd = 0;
  while (is < ns || itd < nt) {
    const bool take_tiled = itd < nt && (is >= ns || itd * ns <= is * nt);
    out.push_back(take_tiled ? qt[itd++] : qs[is++]);
  }
}

// The order of a mixed launch.  Workgroup i of a launch runs on XCD i %
// kXcds (measured on MI355X for every workgroup of a launch), and each XCD
// has its own L2: the tiled row blocks of one (sequence, KV head) read the
// same K/V tiles, so they are kept on one XCD (its L2 then fetches those
// tiles once, not once per XCD).  Groups go to the XCD with the least tiled
// work so far, largest groups first; small-row items, longest first, fill
// each XCD's queue up to an equal share of the launch, least-loaded XCD
// first; each queue is merged in proportion; the queues are interleaved so
// that position p holds an item of queue p % kXcds (a queue that runs out
// early lends its slots to the longest one).
constexpr int kXcds = 8;
void emit_mixed(const std::vector<Item>& small, const std::vector<Item>& tiled, int32_t num_kv_heads,
                int32_t* dst) {
  // thread-local buffers that keep their capacity between calls, bound once
  // to references (each access to a thread_local of a shared library may
  // cost a TLS lookup)
  thread_local std::vector<uint32_t> os_tls, ot_tls;
  thread_local std::vector<int32_t> gid_tls, gkey_tls, gorder_tls;
  thread_local std::vector<int64_t> gcost_tls;
  thread_local std::vector<int8_t> gxcd_tls;
  thread_local std::vector<const Item*> qt_tls[kXcds], qs_tls[kXcds], q_tls[kXcds];
  std::vector<uint32_t>& os = os_tls;
  std::vector<uint32_t>& ot = ot_tls;
  std::vector<int32_t>& gid_of_key = gid_tls;
  std::vector<int32_t>& gkey = gkey_tls;
  std::vector<int32_t>& gorder = gorder_tls;
  std::vector<int64_t>& gcost = gcost_tls;
  std::vector<int8_t>& gxcd = gxcd_tls;
  std::vector<const Item*>* qt = qt_tls;
  std::vector<const Item*>* qs = qs_tls;
  std::vector<const Item*>* q = q_tls;
  order_by_cost(small, os);
  order_by_cost(tiled, ot);
  // tiled groups (sequence x KV heads + KV head), numbered in order of first
  // appearance in the longest-first list
  int32_t max_seq = 0;
  for (const Item& it : tiled) max_seq = std::max(max_seq, it.w[0]);
  gid_of_key.assign((size_t)(max_seq + 1) * num_kv_heads, -1);
  gkey.clear();
  gcost.clear();
  for (uint32_t i : ot) {
    const int32_t key = tiled[i].w[0] * num_kv_heads + tiled[i].w[1];
    if (gid_of_key[key] < 0) {
      gid_of_key[key] = (int32_t)gcost.size();
      gkey.push_back(key);
      gcost.push_back(0);
    }
    gcost[gid_of_key[key]] += tiled[i].cost;
  }
  gorder.resize(gcost.size());
  for (size_t g = 0; g < gorder.size(); ++g) gorder[g] = (int32_t)g;
  std::stable_sort(gorder.begin(), gorder.end(),
                   [&gcost](int32_t a, int32_t b) { return gcost[a] > gcost[b]; });
  int64_t work[kXcds] = {};
  gxcd.resize(gcost.size());
  for (int32_t g : gorder) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (work[x] < work[best]) best = x;
    gxcd[g] = (int8_t)best;
    work[best] += gcost[g];
  }
  for (int x = 0; x < kXcds; ++x) {
    qt[x].clear();
    qs[x].clear();
    q[x].clear();
  }
  for (uint32_t i : ot) {
    const int32_t key = tiled[i].w[0] * num_kv_heads + tiled[i].w[1];
    qt[gxcd[gid_of_key[key]]].push_back(&tiled[i]);
  }
  const size_t total = small.size() + tiled.size();
  for (uint32_t i : os) {
    int best = -1;
    for (int x = 0; x < kXcds; ++x) {
      const size_t cap = total / kXcds + ((size_t)x < total % kXcds ? 1 : 0);
      if (qt[x].size() + qs[x].size() >= cap) continue;
      if (best < 0 || work[x] < work[best]) best = x;
    }
    if (best < 0) {   // every queue at its share (tiled groups overfilled some)
      best = 0;
      for (int x = 1; x < kXcds; ++x)
        if (qt[x].size() + qs[x].size() < qt[best].size() + qs[best].size()) best = x;
    }
    qs[best].push_back(&small[i]);
    work[best] += small[i].cost;
  }
  for (int x = 0; x < kXcds; ++x) merge_proportional(qs[x], qt[x], q[x]);
  size_t head[kXcds] = {};
  for (size_t pos = 0; pos < total; ++pos) {
    int x = (int)(pos % kXcds);
    if (head[x] == q[x].size()) {   // lend the slot to the queue with the most left
      int best = -1;
      for (int y = 0; y < kXcds; ++y)
        if (head[y] < q[y].size() && (best < 0 || q[y].size() - head[y] > q[best].size() - head[best]))
          best = y;
      x = best;
    }
    std::memcpy(dst, q[x][head[x]++]->w, sizeof(Item::w));
    dst += PA_ITEM_WORDS;
  }
}

}  // namespace

pa_status plan(const pa_attn_params* p, const int32_t* cu, const int32_t* sk,
               int32_t force_splits, int32_t* wl, size_t cap, pa_plan_info* info) {
  pa_status st = check_params(p);
  if (st != PA_OK) return st;
  if (!info) return PA_ERR_INVALID_ARGUMENT;
  if (p->batch > 0 && (!cu || !sk)) return PA_ERR_INVALID_ARGUMENT;
  if (force_splits < 0) return PA_ERR_INVALID_ARGUMENT;
  const int32_t B = p->batch, H = p->num_heads, Hkv = p->num_kv_heads;
  const int32_t G = H / Hkv;
  const int64_t max_k = (int64_t)p->max_blocks_per_seq * p->block_size;
  if (B > 0 && cu[0] != 0) return PA_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < B; ++b) {
    if (cu[b + 1] < cu[b]) return PA_ERR_INVALID_ARGUMENT;
    if (sk[b] < 0 || sk[b] > max_k) return PA_ERR_INVALID_ARGUMENT;
    // rows of one sequence are indexed in 32 bits
    if ((int64_t)(cu[b + 1] - cu[b]) * G > INT32_MAX / 2) return PA_ERR_INVALID_ARGUMENT;
  }
  const int32_t T = B > 0 ? cu[B] : 0;
  if ((int64_t)T * H > INT32_MAX) return PA_ERR_INVALID_ARGUMENT;

  // ---- units: (seq, kvh, row block) with their visible key range.  The
  // vectors are per thread and keep their capacity between calls: the planner
  // runs once per step on the host, and allocation would dominate its cost.
  thread_local std::vector<Unit> units;
  units.clear();
  // Tiled row blocks: PA_TILED_ROWS_WIDE rows (8-wave workgroups sharing each
  // K/V tile) when no sequence is small-row, D <= 128, and either D = 64 or
  // the prefills are long (2048 query tokens or more on average) and the
  // cache is not one that the DMA kernel runs (bf16 at D = 128 with a
  // power-of-two block size); else PA_TILED_ROWS (4-wave workgroups).
  // Measured on MI355X (H = 32, Hkv = 8, causal): with register-staged tile
  // loads 256-row blocks took 4-9 % less time for prefills of 2048-8192
  // tokens and 3 % less at D = 64 for 256-2048 tokens; with DMA tile loads
  // 128-row blocks in 4-wave workgroups were faster at every length (3 % on
  // 4 x 8192 tokens, 4-8 % on 592-1811 tokens, measured at two workgroups
  // per compute unit; they now run three).
  bool any_small = false;
  int64_t tiled_q = 0, tiled_seqs = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t Lq = cu[b + 1] - cu[b];
    if (Lq == 0) continue;
    if (Lq * G <= PA_SMALL_MAX_ROWS) {
      any_small = true;
    } else {
      tiled_q += Lq;
      ++tiled_seqs;
    }
  }
  const bool dma_kernel = p->head_size == 128 && !p->kv_cache_fp8 &&
                          (p->block_size & (p->block_size - 1)) == 0;
  const bool wide = !any_small && tiled_seqs > 0 && p->head_size <= 128 &&
                    (p->head_size <= 64 || (tiled_q >= 2048 * tiled_seqs && !dma_kernel));
  const int32_t tiled_rows = wide ? PA_TILED_ROWS_WIDE : PA_TILED_ROWS;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t Lq = cu[b + 1] - cu[b], Lk = sk[b];
    if (Lq == 0) continue;
    const int32_t R = Lq * G;
    const bool small = R <= PA_SMALL_MAX_ROWS;
    const int32_t rb = small ? R : tiled_rows;
    for (int32_t kvh = 0; kvh < Hkv; ++kvh)
      for (int32_t r0 = 0; r0 < R; r0 += rb) {
        const int32_t nr = std::min(rb, R - r0);
        int64_t kv_end = Lk;
        if (p->causal) {
          // bottom-right alignment: the block's last query token i sees keys
          // j <= i + Lk - Lq
          const int64_t i_last = (r0 + nr - 1) / G;
          kv_end = std::min<int64_t>(Lk, std::max<int64_t>(0, i_last + Lk - Lq + 1));
        }
        int64_t kv_begin = 0;
        if (p->sliding_window > 0) {
          // the block's first query token i sees keys j >= i + Lk - Lq - (W - 1);
          // ranges start on a multiple of 16 (one cache block per 16 keys)
          const int64_t i_first = r0 / G;
          const int64_t lo = i_first + Lk - Lq - (p->sliding_window - 1);
          kv_begin = std::min<int64_t>(std::max<int64_t>(lo, 0), kv_end) / 16 * 16;
        }
        units.push_back(Unit{b, kvh, r0, nr, (int32_t)kv_end, small, (int32_t)kv_begin});
      }
  }

  // ---- split-KV choice
  int64_t small_keys = 0, tiled_keys = 0, n_tiled = 0, n_small = 0;
  for (const Unit& u : units) {
    if (u.small) { small_keys += u.kv_end - u.kv_begin; ++n_small; }
    else { tiled_keys += u.kv_end - u.kv_begin; ++n_tiled; }
  }
  // compute units to fill: the caller's device, or one whole MI355X
  const int64_t target = p->num_cus > 0 ? p->num_cus : PA_PLAN_TARGET_CUS;
  int64_t tiled_chunk = 0;
  // tiled rows (bound by the matrix cores): split only when there are too
  // few blocks to fill the chip; cuts fall on whole key tiles
  if (force_splits == 0 && n_tiled > 0 && n_tiled < target) {
    const int64_t want_t = 2 * target;
    tiled_chunk = std::max<int64_t>(kTiledMinChunk,
                                    ceil_div(ceil_div(std::max<int64_t>(tiled_keys, 1), want_t),
                                             kKeyTile) * kKeyTile);
  }

  thread_local std::vector<Item> small_items, tiled_items, reduce_items;
  small_items.clear();
  tiled_items.clear();
  reduce_items.clear();
  int64_t prow = 0;
  // Lk - Lq of a unit's sequence
  auto koff = [&](const Unit& u) { return sk[u.seq] - (cu[u.seq + 1] - cu[u.seq]); };
  // a unit whose range became items [first, end) of `dst`: when it is split,
  // give every piece its partial rows and add the reduce item
  auto finish_unit = [&](const Unit& u, std::vector<Item>& dst, size_t first) -> bool {
    const int64_t n = (int64_t)(dst.size() - first);
    if (n <= 1) return true;
    for (int64_t s = 0; s < n; ++s) dst[first + s].w[6] = (int32_t)(prow + s * u.nrows);
    reduce_items.push_back(
        Item{{u.seq, u.kvh, u.row0, u.nrows, (int32_t)prow, (int32_t)n, cu[u.seq], 0, 0, 0, 0, 0}, 0});
    prow += n * u.nrows;
    return prow <= INT32_MAX / 2;
  };

  // ---- small units (HBM-bound): cut into pieces so that there are about
  // kSmallItemsPerCu workgroups per CU (each piece a multiple of 64 keys:
  // one step of every wave, never under kSmallMinChunk); forced splits
  // (tests) cut every unit into force_splits ranges of a multiple of 16 keys
  if (n_small > 0) {
    const int64_t chunk = std::max<int64_t>(
        kSmallMinChunk,
        ceil_div(ceil_div(std::max<int64_t>(small_keys, 1),
                          (int64_t)(target * (p->head_size >= 256 ? kSmallItemsPerCuD256
                                              : p->kv_cache_fp8 && n_tiled == 0
                                                  ? kSmallItemsPerCuFp8
                                              : dma_kernel && n_tiled > 0
                                                  ? kSmallItemsPerCuDmaMix
                                                  : kSmallItemsPerCu))),
                 64) * 64);
    for (const Unit& u : units) {
      if (!u.small) continue;
      const size_t first = small_items.size();
      const int32_t kv = u.kv_end - u.kv_begin;
      int32_t c = kv;
      if (kv > 0) {
        if (force_splits > 0) {
          c = std::max(16, ceil_div32(ceil_div32(kv, force_splits), 16) * 16);
        } else if (kv > chunk) {
          const int32_t nsp = ceil_div32(kv, (int32_t)chunk);
          c = ceil_div32(ceil_div32(kv, nsp), 64) * 64;
        }
      }
      // in a mixed launch of the LDS-DMA kernel a split unit's last piece is
      // cut finer (kSmallTailCutsMixed pieces), so that the longest-first
      // order ends on short items and the launch drains faster
      const bool graded = force_splits == 0 && kv > chunk && dma_kernel && n_tiled > 0;
      const int32_t tail_cuts = kSmallTailCutsMixed;
      int32_t k0 = u.kv_begin;
      int32_t step = std::max(c, 1);
      do {   // (an empty range still gets its item: its rows are written)
        int32_t k1 = std::min(u.kv_end, k0 + step);
        if (graded && k1 == u.kv_end && step == c && k1 - k0 >= 128) {
          const int32_t q = std::min(tail_cuts, (k1 - k0) / 64);
          step = ceil_div32(ceil_div32(k1 - k0, q), 64) * 64;
          k1 = std::min(u.kv_end, k0 + step);
        }
        // cost: an estimate of the workgroup's time, comparable with the
        // tiled items' (a small-row workgroup streams a key about as fast as
        // a full 128-row tiled one computes it)
        small_items.push_back(
            Item{{u.seq, u.kvh, u.row0, u.nrows, k0, k1, -1, 0, cu[u.seq], koff(u), 0, 0},
                 (int64_t)(k1 - k0) * PA_TILED_ROWS});
        k0 = k1;
      } while (k0 < u.kv_end);
      if (!finish_unit(u, small_items, first)) return PA_ERR_INVALID_ARGUMENT;
    }
  }

  // ---- tiled units
  for (const Unit& u : units) {
    if (u.small) continue;
    // planner-chosen cuts fall on whole key tiles; forced splits (tests)
    // only keep ranges a multiple of 16 keys so tiny inputs still split
    // (32-bit arithmetic: key counts are below 2^30, and 64-bit divisions
    // would dominate the planner's time)
    const int32_t align = force_splits > 0 ? 16 : kKeyTile;
    const int32_t kv = u.kv_end - u.kv_begin;
    int32_t chunk = kv;
    if (kv > 0) {
      if (force_splits > 0) {
        chunk = ceil_div32(ceil_div32(kv, force_splits), align) * align;
      } else if (tiled_chunk > 0 && kv > tiled_chunk) {
        // equal-sized pieces, each a multiple of the alignment
        const int32_t n = ceil_div32(kv, (int32_t)tiled_chunk);
        chunk = ceil_div32(ceil_div32(kv, n), align) * align;
      }
      chunk = std::max(chunk, align);
    }
    const size_t first = tiled_items.size();
    int32_t k0 = u.kv_begin;
    do {
      const int32_t k1 = std::min(u.kv_end, k0 + chunk);
      tiled_items.push_back(
          Item{{u.seq, u.kvh, u.row0, u.nrows, k0, k1, -1, 1, cu[u.seq], koff(u), 0, 0},
               (int64_t)(k1 - k0) * u.nrows});
      k0 = k1;
    } while (k0 < u.kv_end);
    if (!finish_unit(u, tiled_items, first)) return PA_ERR_INVALID_ARGUMENT;
  }
  const size_t n_items = small_items.size() + tiled_items.size() + reduce_items.size();
  const size_t words = PA_WORKLIST_HEADER_WORDS + n_items * PA_ITEM_WORDS;
  info->num_small_items = (int32_t)small_items.size();
  info->num_tiled_items = (int32_t)tiled_items.size();
  info->num_reduce_items = (int32_t)reduce_items.size();
  info->num_partial_rows = (int32_t)prow;
  info->max_reduce_rows = 0;
  for (const Item& it : reduce_items) info->max_reduce_rows = std::max(info->max_reduce_rows, it.w[3]);
  info->batch = B;
  info->num_heads = H;
  info->num_kv_heads = Hkv;
  info->head_size = p->head_size;
  info->causal = p->causal;
  info->sliding_window = p->sliding_window;
  info->tiled_rows = tiled_rows;
  info->num_tokens = T;
  info->worklist_bytes = words * sizeof(int32_t);
  // partial rows: fp32 [prow, D] values, then fp32 [prow] lse, 256-B aligned
  const size_t o_bytes = (size_t)prow * p->head_size * sizeof(float);
  const size_t l_bytes = (size_t)prow * sizeof(float);
  info->workspace_bytes = prow ? ((o_bytes + 255) / 256 * 256 + (l_bytes + 255) / 256 * 256) : 0;
  if (!wl) return PA_OK;
  if (cap < info->worklist_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
  std::memset(wl, 0, PA_WORKLIST_HEADER_WORDS * sizeof(int32_t));
  wl[0] = PA_WORKLIST_MAGIC;
  wl[1] = PA_WORKLIST_VERSION;
  wl[2] = info->num_small_items;
  wl[3] = info->num_tiled_items;
  wl[4] = info->num_reduce_items;
  wl[5] = info->num_partial_rows;
  wl[6] = G;
  wl[7] = p->causal;
  // longest work first, so the tail of the launch is short items; equal
  // costs keep the (seq, kv head) order, which keeps a sequence's blocks
  // close in time and their keys warm in L2
  int32_t* dst = wl + PA_WORKLIST_HEADER_WORDS;
  if (!small_items.empty() && !tiled_items.empty()) {
    // one mixed launch: per XCD, each kind longest first, merged in
    // proportion to their counts (measured on chunked_prefill_mix before the
    // XCD queues: 194 us against 208 us for one merged longest-first order,
    // 215 us small items first, 232 us tiled first)
    emit_mixed(small_items, tiled_items, Hkv, dst);
    dst += (small_items.size() + tiled_items.size()) * PA_ITEM_WORDS;
  } else {
    dst = emit_by_cost(small_items, dst);
    dst = emit_by_cost(tiled_items, dst);
  }
  for (const Item& it : reduce_items) {
    std::memcpy(dst, it.w, sizeof(it.w));
    dst += PA_ITEM_WORDS;
  }
  return PA_OK;
}

}  // namespace pa

extern "C" {

const int32_t pa_supported_head_sizes[PA_NUM_HEAD_SIZES] = {64, 128, 256};

const char* pa_status_str(pa_status s) {
  // callers may pass any int; it is read as one (loading a C++ enum whose
  // value lies outside its enumerators' range is undefined behaviour)
  static_assert(sizeof(pa_status) == sizeof(int32_t), "pa_status is passed as an int");
  int32_t code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
  }
  return "PA_ERR_UNKNOWN";
}

int32_t pa_version(void) { return (5 << 16) | 0; }

pa_status pa_plan_varlen(const pa_attn_params* p, const int32_t* host_cu_seqlens_q,
                         const int32_t* host_seqused_k, int32_t force_splits,
                         int32_t* host_worklist, size_t worklist_capacity_bytes,
                         pa_plan_info* info) {
  return pa::plan(p, host_cu_seqlens_q, host_seqused_k, force_splits, host_worklist,
                  worklist_capacity_bytes, info);
}

pa_status pa_cascade_decide(const pa_attn_params* p, const int32_t* cu, const int32_t* sk,
                            const int32_t* bt, int32_t kv_bytes_per_elem,
                            int32_t* common_prefix_len, int32_t* use_cascade) {
  pa_status st = pa::check_params(p);
  if (st != PA_OK) return st;
  if (!common_prefix_len || !use_cascade) return PA_ERR_INVALID_ARGUMENT;
  if (kv_bytes_per_elem != 1 && kv_bytes_per_elem != 2) return PA_ERR_INVALID_ARGUMENT;
  *common_prefix_len = 0;
  *use_cascade = 0;
  const int32_t B = p->batch;
  if (B > 0 && (!cu || !sk || !bt)) return PA_ERR_INVALID_ARGUMENT;
  if (B > 0 && cu[0] != 0) return PA_ERR_INVALID_ARGUMENT;
  const int32_t BS = p->block_size;
  const int32_t stride = p->block_table_stride ? p->block_table_stride : p->max_blocks_per_seq;
  // the prefix may cover only keys that every query token comes after
  int64_t limit = INT64_MAX;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t Lq = cu[b + 1] - cu[b];
    if (Lq < 0 || sk[b] < 0 || sk[b] > (int64_t)p->max_blocks_per_seq * BS)
      return PA_ERR_INVALID_ARGUMENT;
    limit = std::min<int64_t>(limit, (int64_t)sk[b] - Lq);
  }
  if (B < 2 || limit < BS) return PA_OK;
  const int64_t max_blocks = limit / BS;
  int64_t nblk = 0;
  for (; nblk < max_blocks; ++nblk) {
    const int32_t phys = bt[nblk];
    bool same = phys >= 0 && phys < p->num_blocks;
    for (int32_t b = 1; same && b < B; ++b) same = bt[(int64_t)b * stride + nblk] == phys;
    if (!same) break;
  }
  const int64_t P = nblk * BS;
  *common_prefix_len = (int32_t)P;
  if (!p->causal || p->sliding_window != 0 || P < 256 || B < 8) return PA_OK;

  // cost model: plan both paths and price their launches with times fitted
  // to MI355X measurements of this library (microseconds)
  const double row_bytes = 2.0 * p->head_size * kv_bytes_per_elem;   // K+V of one key, one KV head
  const double kv_heads = p->num_kv_heads;
  // the single pass reads the shared blocks once per sequence; all but the
  // first read come from the last-level cache while the prefix fits in it
  const double prefix_bytes = (double)P * row_bytes * kv_heads;
  const double reread_bw = prefix_bytes <= 128e6 ? 13.6e6 : 6.5e6;   // bytes per us
  double t_single = 0, t_prefix = 0, t_suffix = 0;
  std::vector<int32_t> scu(2), ssk(B), pcu(2), psk(1);
  pa_attn_params pp, sp;
  int32_t col0 = 0;
  st = pa_cascade_split(p, (int32_t)P, cu, sk, &pp, &sp, pcu.data(), psk.data(), ssk.data(), &col0);
  if (st != PA_OK) return st;
  double t_pass[3];
  const pa_attn_params* ps[3] = {p, &pp, &sp};
  const int32_t* cus[3] = {cu, pcu.data(), cu};
  const int32_t* sks[3] = {sk, psk.data(), ssk.data()};
  for (int k = 0; k < 3; ++k) {
    pa_plan_info info;
    st = pa_plan_varlen(ps[k], cus[k], sks[k], 0, nullptr, 0, &info);
    if (st != PA_OK) return st;
    std::vector<int32_t> wl(info.worklist_bytes / 4);
    st = pa_plan_varlen(ps[k], cus[k], sks[k], 0, wl.data(), info.worklist_bytes, &info);
    if (st != PA_OK) return st;
    const int32_t* it = wl.data() + PA_WORKLIST_HEADER_WORDS;
    double small_keys = 0;
    int64_t max_tiled_keys = 0;
    for (int32_t i = 0; i < info.num_small_items + info.num_tiled_items; ++i, it += PA_ITEM_WORDS) {
      const int64_t keys = std::max(0, it[5] - it[4]);
      if (it[7] == 0) small_keys += (double)keys;
      else max_tiled_keys = std::max(max_tiled_keys, keys);
    }
    double t = 0;
    if (info.num_small_items > 0) {
      double bytes = small_keys * row_bytes;
      if (k == 0) {
        // the repeated reads of the shared blocks
        const double reread = (double)(B - 1) * P * kv_heads * row_bytes;
        bytes -= reread;
        t += reread / reread_bw;
      }
      t += 7.8 + bytes / 6.5e6;
    }
    if (info.num_tiled_items > 0)
      t += 10.8 + 1.15 * (double)((max_tiled_keys + 63) / 64) *
                      (double)((info.num_tiled_items + 511) / 512);
    if (info.num_reduce_items > 0) t += 4.2;
    t_pass[k] = t;
  }
  t_single = t_pass[0];
  t_prefix = t_pass[1];
  t_suffix = t_pass[2];
  const double t_merge = 3.4;
  *use_cascade = (t_prefix + t_suffix + t_merge < t_single) ? 1 : 0;
  return PA_OK;
}

pa_status pa_cascade_split(const pa_attn_params* p, int32_t common_prefix_len,
                           const int32_t* cu, const int32_t* sk, pa_attn_params* prefix_p,
                           pa_attn_params* suffix_p, int32_t* prefix_cu, int32_t* prefix_sk,
                           int32_t* suffix_sk, int32_t* col0) {
  pa_status st = pa::check_params(p);
  if (st != PA_OK) return st;
  if (!prefix_p || !suffix_p || !prefix_cu || !prefix_sk || !col0) return PA_ERR_INVALID_ARGUMENT;
  if (p->batch > 0 && (!cu || !sk || !suffix_sk)) return PA_ERR_INVALID_ARGUMENT;
  if (p->causal != 1 || p->sliding_window != 0) return PA_ERR_INVALID_ARGUMENT;
  const int32_t BS = p->block_size;
  if (common_prefix_len <= 0 || common_prefix_len % BS != 0) return PA_ERR_INVALID_ARGUMENT;
  const int32_t nblk = common_prefix_len / BS;
  if (nblk >= p->max_blocks_per_seq + 1) return PA_ERR_INVALID_ARGUMENT;
  if (p->batch > 0 && cu[0] != 0) return PA_ERR_INVALID_ARGUMENT;
  for (int32_t b = 0; b < p->batch; ++b) {
    const int32_t Lq = cu[b + 1] - cu[b];
    if (Lq < 0 || sk[b] < 0) return PA_ERR_INVALID_ARGUMENT;
    // every query token of every sequence lies after the shared prefix
    if ((int64_t)common_prefix_len > (int64_t)sk[b] - Lq) return PA_ERR_INVALID_ARGUMENT;
  }
  const int32_t stride = p->block_table_stride ? p->block_table_stride : p->max_blocks_per_seq;
  const int32_t T = p->batch > 0 ? cu[p->batch] : 0;
  *prefix_p = *p;
  prefix_p->batch = 1;
  prefix_p->max_blocks_per_seq = nblk;
  prefix_p->block_table_stride = stride;
  prefix_p->causal = 0;
  *suffix_p = *p;
  suffix_p->max_blocks_per_seq = std::max(1, p->max_blocks_per_seq - nblk);
  suffix_p->block_table_stride = stride;
  prefix_cu[0] = 0;
  prefix_cu[1] = T;
  prefix_sk[0] = common_prefix_len;
  for (int32_t b = 0; b < p->batch; ++b) suffix_sk[b] = sk[b] - common_prefix_len;
  *col0 = nblk;
  return PA_OK;
}

}  // extern "C"
