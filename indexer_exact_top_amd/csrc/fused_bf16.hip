// Fused Indexer-TopK instantiations with bf16 queries (bf16 or e4m3fn keys).
#include "fused_qrow.hpp"

namespace itk {
FusedLauncher find_fused_launcher_bf16(int qt, int kt, int hb, int d, bool relu, bool q8)
{
    ITK_FUSED_Q8_CASES_FOR(ITK_BF16)
    ITK_FUSED_CASES_FOR(ITK_BF16, ITK_BF16)
    ITK_FUSED_CASES_FOR(ITK_BF16, ITK_FP8_E4M3)
    return nullptr;
}
FusedLauncher find_qrow_launcher_bf16(int qt, int kt, int d, bool relu)
{
    ITK_QROW_CASES_FOR(ITK_BF16, ITK_BF16)
    ITK_QROW_CASES_FOR(ITK_BF16, ITK_FP8_E4M3)
    return nullptr;
}
}  // namespace itk
