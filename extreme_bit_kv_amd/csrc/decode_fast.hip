// Placeholder: the MFMA decode kernel is not built yet.
#include "cq_internal.h"
namespace cqi {
size_t decode_fast_ws(int, int, int, int, int, int) { return 0; }
bool decode_fast_supported(const DecodeArgs&) { return false; }
hipError_t decode_fast(const DecodeArgs&) { return hipErrorNotSupported; }
}  // namespace cqi
