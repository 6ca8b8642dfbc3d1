// Fused Indexer-TopK instantiations with fp32 queries and keys.
#include "fused_impl.hpp"

namespace itk {
FusedLauncher find_fused_launcher_f32(int qt, int kt, int hb, int d, bool relu, bool q8)
{
    if (q8) return nullptr;
    ITK_FUSED_CASES_F32
    return nullptr;
}
}  // namespace itk
