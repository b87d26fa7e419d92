// BF16 instantiations of the multi-query MFMA kernel (see multi_query_mfma.h).
#include "multi_query_mfma.h"

namespace pa {

int launch_multi_query_bf16(const DecodeArgs &a) { return mq::by_dim<BF16>(a); }

}  // namespace pa
