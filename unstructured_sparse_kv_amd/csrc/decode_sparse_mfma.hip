// Group-size dispatch of the matrix-core sparse decode kernels
// (decode_sparse_mfma.hpp; one translation unit per group size).
#include "kernels.hpp"

namespace mustafar {

hipError_t launch_decode_sparse_g1(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_sparse_g2(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_sparse_g4(const SparseDecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_sparse_g8(const SparseDecodeArgs& a, int batch, hipStream_t stream);

hipError_t launch_decode_sparse(const SparseDecodeArgs& a, int batch, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_decode_sparse_g1(a, batch, stream);
    case 2: return launch_decode_sparse_g2(a, batch, stream);
    case 4: return launch_decode_sparse_g4(a, batch, stream);
    case 8: return launch_decode_sparse_g8(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mustafar
