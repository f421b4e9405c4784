#include "launch.h"
namespace mla {
bool mfma_attn_supported(const AttnCall &, const char **why) { *why = "not built"; return false; }
size_t mfma_attn_workspace(const AttnCall &) { return 0; }
int32_t mfma_attn_splits(const AttnCall &, int) { return 1; }
hipError_t mfma_absorb_attn(const AttnCall &) { return hipErrorNotSupported; }
}
