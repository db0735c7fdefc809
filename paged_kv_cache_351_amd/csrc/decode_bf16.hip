// Decode-attention instantiations for one element type (see decode_kernel.h).
#include "decode_kernel.h"

namespace pagedkv {

bool decode_kernels_bf16(int head_dim, int block_size, int gp, DecodeVariant variant, const void** dec,
                        const void** red) {
  return pick_decode_kernels<kBF16>(head_dim, block_size, gp, variant, dec, red);
}

}  // namespace pagedkv
