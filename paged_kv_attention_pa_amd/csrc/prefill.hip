// Varlen prefill (placeholder until the MFMA kernel lands).
#include "launch.hpp"
namespace pa {
hipError_t launch_prefill_varlen(const PrefillVarlen&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pa
