#include "launch.h"
namespace mla {
bool mfma_expand_supported(const ExpandCall &, const char **why) { *why = "not built"; return false; }
hipError_t mfma_expand_kv(const ExpandCall &) { return hipErrorNotSupported; }
}
