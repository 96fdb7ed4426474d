// mustafar_decode_attn / mustafar_decode_step kernels for 4 query heads per kv
// head (one translation unit per group size, so the instantiations build in parallel).
#include "decode_sparse_mfma.hpp"

namespace mustafar {

hipError_t launch_decode_sparse_g4(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  return launch_mfma_g<4>(a, batch, stream);
}

}  // namespace mustafar
