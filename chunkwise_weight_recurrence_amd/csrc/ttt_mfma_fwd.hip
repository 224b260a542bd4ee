// Matrix-core (bf16 MFMA) forward of the chunkwise TTT layer -- not yet enabled.
#include "ttt_internal.h"
namespace ttt {
bool mfma_fwd_supported(const FwdArgs&) { return false; }
size_t mfma_fwd_workspace(const FwdArgs&) { return 0; }
hipError_t mfma_fwd_launch(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
bool mfma_bwd_supported(const BwdArgs&) { return false; }
size_t mfma_bwd_workspace(const BwdArgs&) { return 0; }
hipError_t mfma_bwd_launch(const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ttt
