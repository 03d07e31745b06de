// Matrix-core split-KV decode (gfx950).  Not yet enabled: the dispatch falls
// back to the generic kernel until this kernel is in place.
#include "qkn_internal.h"

namespace qkn {

bool mfma_decode_supported(const qkn_mla_dims&) { return false; }

hipError_t launch_decode_mfma(const qkn_mla_dims&, const DecodeArgs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace qkn
