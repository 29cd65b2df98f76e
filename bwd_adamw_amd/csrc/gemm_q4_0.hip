// bf16 GEMM and row-pass instances for Q4_0 frozen W (a translation unit of its own).
#define LORA_WQ_INSTANCES
#include "gemm_wq.hpp"

namespace lora {
template void launch_gemm_wq_tiles<WQ_Q4_0>(int, bool, bool, dim3, hipStream_t,
                                            const prof::Scope&, const GemmBf16Args&);
template void launch_row_pass_wq<WQ_Q4_0>(int, bool, int, bool, dim3, hipStream_t, const prof::Scope&,
                                          const RowPassArgs&);
}  // namespace lora
