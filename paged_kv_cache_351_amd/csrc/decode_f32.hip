// Decode-attention instantiations for one element type (see decode_kernel.h).
#include "decode_kernel.h"

namespace pagedkv {

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t stream) {
  return dispatch_decode<kF32>(p, stream);
}

}  // namespace pagedkv
