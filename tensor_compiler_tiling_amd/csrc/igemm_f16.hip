// fp16 / bf16 implicit-GEMM convolution on CDNA4 matrix cores (registry).
#include "ct_device.hpp"
#include "igemm_common.hpp"

namespace ct {

const IgemmVariant* igemm_f16_variants(int* count) {
    static const IgemmVariant kNone[1] = {};
    *count = 0;
    return kNone;
}

}  // namespace ct
