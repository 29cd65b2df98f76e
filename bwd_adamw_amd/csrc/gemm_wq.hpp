// Launch of the block-quantized-W instances of the bf16 GEMM and of the row
// pass (DoRA norms, merge).  Each format's instances live in a translation
// unit of their own (gemm_q*.hip), so that the library's objects compile in
// parallel.
#pragma once
#include "gemm_bf16.hpp"
#include "launch.hpp"
#include "rowpass.hpp"

namespace lora {

// Tile configuration `cfg` (LORA_BF16_CFGS) of the product in direction
// `fwd`, for W in format WQ; `exact` as for the bf16 instances.
template <int WQ>
void launch_gemm_wq_tiles(int cfg, bool fwd, bool exact, dim3 grid, hipStream_t st,
                          const prof::Scope& ps, const GemmBf16Args& a);

// The row pass over W in format WQ: mode 0 DoRA norms, 1 merge (bf16 or
// float32 output); lora_on adds s B A at padded rank rp.
template <int WQ>
void launch_row_pass_wq(int mode, bool lora_on, int rp, bool out_bf16, dim3 grid, hipStream_t st,
                        const prof::Scope& ps, const RowPassArgs& a);

#ifdef LORA_WQ_INSTANCES
template <int WQ>
void launch_row_pass_wq(int mode, bool lora_on, int rp, bool out_bf16, dim3 grid, hipStream_t st,
                        const prof::Scope& ps, const RowPassArgs& a) {
#define LORA_WQ_ROWS(RP_, LORA_)                                                               \
  if (mode == 0) launch(row_pass_kernel<uint8_t, RP_, LORA_, 0, float, WQ>, grid, st, ps, a);   \
  else if (out_bf16) launch(row_pass_kernel<uint8_t, RP_, LORA_, 1, uint16_t, WQ>, grid, st, ps, a); \
  else launch(row_pass_kernel<uint8_t, RP_, LORA_, 1, float, WQ>, grid, st, ps, a);
  if (!lora_on) { LORA_WQ_ROWS(16, false) }
  else if (rp <= 16) { LORA_WQ_ROWS(16, true) }
  else if (rp <= 32) { LORA_WQ_ROWS(32, true) }
  else if (rp <= 64) { LORA_WQ_ROWS(64, true) }
  else { LORA_WQ_ROWS(128, true) }
#undef LORA_WQ_ROWS
}

template <int WQ>
void launch_gemm_wq_tiles(int cfg, bool fwd, bool exact, dim3 grid, hipStream_t st,
                          const prof::Scope& ps, const GemmBf16Args& a) {
#define LORA_WQ_TILE(i, BM_, BN_, NT_, WGM_, BK_, D_, DIRS_, AF_, BF_, AD_, BD_)                \
  if (cfg == i) {                                                                             \
    if constexpr (D_ == 0) {                                                                  \
      /* the direct-operand loop takes bf16 W only; the planner never picks it here */       \
    } else if (fwd) {                                                                         \
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
