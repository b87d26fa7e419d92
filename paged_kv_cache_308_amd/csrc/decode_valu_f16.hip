// F16 instantiations of the vector-ALU decode kernels (see decode_valu.h).
#include "decode_valu.h"

namespace pa {

int launch_decode_valu_f16(const DecodeArgs &a) { return valu::by_dim<valu::SameKV<F16>>(a); }
int launch_lse_merge_f16(const DecodeArgs &a) { return valu::merge_dim<F16>(a); }

}  // namespace pa
