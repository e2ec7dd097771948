// Placeholder: the fused single-read quantization kernel is not built yet.
#include "cq_internal.h"
namespace cqi {
size_t quant_fused_ws(int, int, int, int) { return 0; }
bool quant_fused_supported(const QuantArgs&) { return false; }
hipError_t quant_fused(const QuantArgs&) { return hipErrorNotSupported; }
}  // namespace cqi
