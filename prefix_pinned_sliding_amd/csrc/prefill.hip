// Chunked-prefill attention on MFMA (K4). Not built yet: the launcher reports an error.
#include "psa_internal.h"

namespace psa {

hipError_t launch_prefill(const DevCache&, const void*, const void*, void*, float*, int, int,
                          hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace psa
