// Instantiations of the sparse expert kernel with the up codes at 8, 4 and 1
// bits (fp16 and bf16 activations).
#include "expert_sparse.hpp"

namespace moeffn {
hipError_t launch_sparse_expert_bits(const SparseArgs &a, int bits, bool bf16, int tb, hipStream_t s)
{
    switch (bits) {
    case 8: return bf16 ? sparse::launch_dtype<true, 8>(a, tb, s) : sparse::launch_dtype<false, 8>(a, tb, s);
    case 4: return bf16 ? sparse::launch_dtype<true, 4>(a, tb, s) : sparse::launch_dtype<false, 4>(a, tb, s);
    case 1: return bf16 ? sparse::launch_dtype<true, 1>(a, tb, s) : sparse::launch_dtype<false, 1>(a, tb, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace moeffn
