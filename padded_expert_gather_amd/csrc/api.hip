// api.hip - library-wide entry points: status names, ABI version, workspace
// size.
#include "peg_host.hpp"

using namespace peg;

PEG_API const char* peg_status_string(peg_status s) {
    switch (s) {
        case PEG_OK: return "ok";
        case PEG_ERR_NULL_ARG: return "a required pointer is NULL";
        case PEG_ERR_BAD_SHAPE: return "a size argument is out of range";
        case PEG_ERR_BAD_DTYPE: return "unsupported dtype or layout code";
        case PEG_ERR_WORKSPACE: return "workspace missing or too small";
        case PEG_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case PEG_ERR_ALIGNMENT: return "a buffer is not aligned to its element size";
        case PEG_ERR_SCRATCH_LIMIT: return "the sizes need more than the library's static scratch";
        default: return "unknown status";
    }
}

PEG_API int32_t peg_abi_version(void) { return (1 << 16) | 0; }

PEG_API size_t peg_workspace_bytes(int64_t T, int32_t K, int32_t E) {
    if (T < 0 || K < 1 || E < 1 || E > PEG_MAX_EXPERTS || T > kMaxAssign / K) return 0;
    return ws_need(T, K, E);
}
