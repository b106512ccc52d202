// Shared between the planner (plan.cpp) and the launchers (pagedattn.hip):
// the tile geometry both sides must agree on.
#ifndef PAGEDATTN_PLAN_INTERNAL_H_
#define PAGEDATTN_PLAN_INTERNAL_H_

#include <cstdint>

#include "pagedattn.h"

namespace pa {

// tiled kernel: 4 waves x 32 rows, key tiles of kKeyTile keys
constexpr int kTiledWaves = 4;
constexpr int kKeyTile = 64;
constexpr int kTiledMinChunk = 256;
// small-row kernel: 4 waves taking 16-key steps in turn; the planner cuts
// key ranges into pieces of at least kSmallMinChunk keys so that there are
// about kSmallItemsPerCu workgroups per compute unit (of 2.5 ... 5, measured
// on MI355X, 3.5 suits the bf16 decode batch and chunked-prefill mixes best)
constexpr int kSmallWaves = 4;
constexpr int kSmallStep = 16;
constexpr int kSmallMinChunk = 256;
constexpr double kSmallItemsPerCu = 3.5;
// at D = 256 one small-row workgroup fits a compute unit (three or four at
// D <= 128): 2.5 measured best of 2 ... 4 on the long-context decode batch
// (16 sequences of 32K-128K keys: 454 us against 464 us at 3.5)
constexpr double kSmallItemsPerCuD256 = 2.5;
// an E4M3 cache halves each piece's bytes and fits four small-row workgroups
// per compute unit at D <= 128: 4.5 measured best of 3.5 ... 5 on the 64-
// sequence decode batch (60.4 us against 62.3 us at 3.5 and 62.0 us at 5).
// Used for launches of small items only: with tiled items beside them (a
// chunked-prefill mix) 3.5 stays faster, 183-185 us against 187-189 us.
constexpr double kSmallItemsPerCuFp8 = 4.5;
// mixed launches of the LDS-DMA kernel (bf16 cache, D = 128, power-of-two
// block size) hold three workgroups per compute unit: 4.5 measured best of
// 3.5 / 4.5 / 5.5 on the chunked-prefill mix (185.2-186.5 us against
// 189.1-189.8 us at 3.5; 5.5 within noise of 4.5)
constexpr double kSmallItemsPerCuDmaMix = 4.5;
// in a mixed launch of the LDS-DMA kernel (bf16 cache, D = 128,
// power-of-two block size) the last piece of a split small-row unit is cut
// into this many: a timestamp probe of the decode batch showed a launch
// draining over its last third, as equal pieces ended unevenly.  Measured
// (HIP events, three runs each): chunked-prefill mix 182.6-183.5 us against
// 185.5-188.5 us.  Launches of small items alone keep whole pieces: 4 cuts
// saved about 1 us of the decode call but doubled its items, and the larger
// work list and plan made the whole step slower (E4M3 decode step 70 -> 79
// us); at D = 256 finer pieces were slower
constexpr int32_t kSmallTailCutsMixed = 2;

static_assert(PA_TILED_ROWS == kTiledWaves * 32, "tiled row block");

pa_status check_params(const pa_attn_params* p);
bool head_size_supported(int32_t d);
pa_status plan(const pa_attn_params* p, const int32_t* cu, const int32_t* sk,
               int32_t force_splits, int32_t* wl, size_t cap, pa_plan_info* info);

}  // namespace pa

#endif  // PAGEDATTN_PLAN_INTERNAL_H_
