// Decode-attention instantiations for one element type (see decode_kernel.h).
#include "decode_kernel.h"

namespace pagedkv {

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  return dispatch_decode<kBF16>(p, stream);
}

}  // namespace pagedkv
