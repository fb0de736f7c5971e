// bf16 MFMA kernel: not built yet.
#include "common.h"
#include "launch.h"

namespace so2 {

bool mfma_supported(int, int, int) { return false; }
size_t mfma_scratch_bytes(int, int, int) { return 0; }
so2_status launch_attention_mfma(const AttnArgs&, hipStream_t) { return SO2_ERR_UNSUPPORTED; }

}  // namespace so2
