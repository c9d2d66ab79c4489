// Matrix-core paged decode attention (bfloat16/float16, block_size 16): not built yet.
#include "launchers.h"

namespace pkv {

int launch_decode_mfma(const DecodeArgs&, const DecodePlan&, int, hipStream_t) { return -1; }

}  // namespace pkv
