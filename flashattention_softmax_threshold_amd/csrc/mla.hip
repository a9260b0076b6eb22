// mla.hip -- MLA-shaped BLASST decode (V = first 512 columns of the 576-wide latent K).
#include "internal.h"

namespace blasst {

hipError_t launch_decode_mla(const DecodeParams &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace blasst
