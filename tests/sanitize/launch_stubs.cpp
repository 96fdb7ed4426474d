// Kernel launchers replaced by stubs for the host-side sanitizer build of the
// library's C ABI (api.hip with the sanitizers on its host side).  The driver only takes
// paths that return before any launch; a stub that is reached reports it.
#include <stdio.h>
#include <stdlib.h>

#include "../../unstructured_sparse_kv_amd/csrc/kernels.hpp"

namespace mustafar {

static hipError_t reached(const char* what) {
  fprintf(stderr, "launch stub reached: %s\n", what);
  abort();
}

hipError_t launch_prune_compress(const mustafar_kv_t&, const KeepMap&, const uint16_t*, int64_t,
                                 const int32_t*, hipStream_t, bool) {
  return reached("prune_compress");
}
hipError_t launch_prune_compress_channel(const mustafar_kv_t&, const KeepMap&, const uint16_t*,
                                         int64_t, const int32_t*, hipStream_t) {
  return reached("prune_compress_channel");
}
hipError_t launch_append(const mustafar_kv_t&, const KeepMap&, const mustafar_kv_t&, const KeepMap&,
                         const uint16_t*, const uint16_t*, int32_t*, uint32_t*, hipStream_t) {
  return reached("append");
}
hipError_t launch_decode_sparse(const SparseDecodeArgs&, int, hipStream_t) { return reached("decode"); }
hipError_t launch_decode_sparse_valu(const SparseDecodeArgs&, int, hipStream_t) {
  return reached("decode_valu");
}
hipError_t launch_decode_24(const SparseDecodeArgs&, int, hipStream_t) { return reached("decode_24"); }
hipError_t launch_decode_dense(const DenseDecodeArgs&, int, hipStream_t) { return reached("dense"); }
hipError_t launch_decode_reduce(const float*, int, int, int, int, uint16_t*, hipStream_t, int32_t*,
                                uint32_t*, int32_t, bool) {
  return reached("reduce");
}
hipError_t launch_zero_u32(uint32_t*, uint64_t, hipStream_t) { return reached("zero"); }
hipError_t launch_stream_read(const void*, uint64_t, uint32_t*, hipStream_t) { return reached("stream_read"); }

}  // namespace mustafar
