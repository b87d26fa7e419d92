// F32 instantiations of the vector-ALU decode kernels (see decode_valu.h).
#include "decode_valu.h"

namespace pa {

int launch_decode_valu_f32(const DecodeArgs &a) { return valu::by_dim<valu::SameKV<F32>>(a); }
int launch_lse_merge_f32(const DecodeArgs &a) { return valu::merge_dim<F32>(a); }

}  // namespace pa
