// bsa.hip -- exhaustive selector (placeholder until the MFMA kernel lands).
#include "pisa_internal.hpp"
namespace pisa {
hipError_t launch_bsa(const BsaArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pisa
