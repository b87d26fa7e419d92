// BF16 instantiations of the vector-ALU decode kernels (see decode_valu.h).
#include "decode_valu.h"

namespace pa {

int launch_decode_valu_bf16(const DecodeArgs &a) { return valu::by_dim<valu::SameKV<BF16>>(a); }
int launch_lse_merge_bf16(const DecodeArgs &a) { return valu::merge_dim<BF16>(a); }

}  // namespace pa
