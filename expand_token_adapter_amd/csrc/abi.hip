// abi.hip -- pure host queries of the C ABI (no device work).
#include "device_common.h"
#include "host_checks.h"

using namespace lora;

extern "C" int lora_abi_version(void) { return LORA_ABI_VERSION; }

extern "C" const char* lora_status_string(int status) {
    switch (status) {
        case LORA_OK: return "ok";
        case LORA_ERR_INVALID_ARG: return "invalid argument (null pointer, size, pitch, alignment or enum)";
        case LORA_ERR_UNSUPPORTED: return "unsupported shape (row lengths and pitches must be multiples of 8)";
        case LORA_ERR_WORKSPACE: return "workspace missing or too small";
        case LORA_ERR_HIP: return "HIP launch failed";
        case LORA_ERR_TOO_LARGE: return "the call needs more than the static scratch of a no-allocation entry point";
        default: return "unknown status";
    }
}

extern "C" size_t lora_segments_sched_elems(int32_t T, int32_t num_adapters) {
    if (T < 0 || num_adapters < 1) return 0;
    return (size_t)SchedLayout::make(T, num_adapters).total;
}
