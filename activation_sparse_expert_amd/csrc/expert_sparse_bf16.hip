// bf16 instantiations of the sparse expert kernel.
#include "expert_sparse.hpp"

namespace moeffn {
hipError_t launch_sparse_expert_bf16(const SparseArgs &a, int tb, hipStream_t s)
{
    return sparse::launch_dtype<true>(a, tb, s);
}
}  // namespace moeffn
