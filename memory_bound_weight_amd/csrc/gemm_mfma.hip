// Matrix-core path of the batched-token product (filled in below).
#include "registry.h"

namespace lin {

void register_gemm_mfma(std::vector<Variant>&) {}

}  // namespace lin
