// Stable (key, value) radix sort for binning bodies into grid cells: the
// library primitive of rocPRIM through hipCUB (LSD radix sort, stable, so the
// bodies of a cell stay in ascending original order and the binning is
// deterministic). Kept in its own translation unit: only this file includes
// the hipCUB headers.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>

#include "kernels.h"

namespace nbk {

hipError_t sort_pairs(void *temp, size_t &temp_bytes, const unsigned *keys_in,
                      unsigned *keys_out, const int *vals_in, int *vals_out, int n, int end_bit,
                      hipStream_t stream)
{
    return hipcub::DeviceRadixSort::SortPairs(temp, temp_bytes, keys_in, keys_out, vals_in,
                                              vals_out, n, 0, end_bit, stream);
}

}  // namespace nbk
