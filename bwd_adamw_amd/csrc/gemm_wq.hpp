// Launch of the bf16 GEMM's block-quantized-W instances.  Each format's
// instances live in a translation unit of their own (gemm_q*.hip), so that
// the library's objects compile in parallel.
#pragma once
#include "gemm_bf16.hpp"
#include "launch.hpp"

namespace lora {

// Tile configuration `cfg` (LORA_BF16_CFGS) of the product in direction
// `fwd`, for W in format WQ; `exact` as for the bf16 instances.
template <int WQ>
void launch_gemm_wq_tiles(int cfg, bool fwd, bool exact, dim3 grid, hipStream_t st,
                          const prof::Scope& ps, const GemmBf16Args& a);

#ifdef LORA_WQ_INSTANCES
template <int WQ>
void launch_gemm_wq_tiles(int cfg, bool fwd, bool exact, dim3 grid, hipStream_t st,
                          const prof::Scope& ps, const GemmBf16Args& a) {
#define LORA_WQ_TILE(i, BM_, BN_, NT_, WGM_, BK_, D_, DIRS_, AF_, BF_, AD_, BD_)                \
  if (cfg == i) {                                                                             \
    if (fwd) {                                                                                \
      if constexpr ((DIRS_)&1) {                                                              \
        if (exact)                                                                            \
          launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, true, true, WQ>, grid,       \
                   (unsigned)NT_, st, ps, a);                                                 \
        else                                                                                  \
          launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, true, false, WQ>, grid,      \
                   (unsigned)NT_, st, ps, a);                                                 \
      }                                                                                       \
    } else {                                                                                  \
      if constexpr ((DIRS_)&2) {                                                              \
        if (exact)                                                                            \
          launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, false, true, WQ>, grid,      \
                   (unsigned)NT_, st, ps, a);                                                 \
        else                                                                                  \
          launch_n(gemm_bf16_kernel<BM_, BN_, NT_, WGM_, BK_, D_, false, false, WQ>, grid,     \
                   (unsigned)NT_, st, ps, a);                                                 \
      }                                                                                       \
    }                                                                                         \
    return;                                                                                   \
  }
  LORA_BF16_CFGS(LORA_WQ_TILE)
#undef LORA_WQ_TILE
}
#endif

}  // namespace lora
