// Vector-ALU decode over E4M3 pools with a f16 query (see decode_valu.h).
#include "decode_valu.h"

namespace pa {

int launch_decode_valu_fp8_f16(const DecodeArgs &a) { return valu::e4m3_by_dim<F16>(a); }

}  // namespace pa
