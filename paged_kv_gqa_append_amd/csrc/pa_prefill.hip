// pa_prefill.hip -- chunked-prefill attention (bf16 MFMA tiles); not built yet.
#include "pa_internal.h"

namespace pa {

hipError_t launch_prefill_attention(const PrefillLaunch &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
