// F16 instantiations of the matrix-core decode kernels (see decode_mfma.h).
#include "decode_mfma.h"

namespace pa {

int launch_decode_mfma_f16(const DecodeArgs &a) { return mfma::by_dim<F16>(a); }
int launch_decode_mfma_grouped_f16(const DecodeArgs &a) { return mfma::launch_grouped<F16>(a); }

}  // namespace pa
