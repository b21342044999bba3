// query.hip - MLA query front end (placeholder until the kernel lands).
#include "mla_internal.h"
namespace mla {
size_t query_workspace_bytes(int32_t batch, int32_t heads) { return (size_t)batch * heads * 128 * 2 + 256; }
hipError_t launch_query(const QueryLaunch&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla
