// MLA decode (placeholder until the MFMA kernel lands).
#include "launch.hpp"
namespace pa {
hipError_t launch_mla_decode(const MlaDecode&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pa
