// ssd.hip -- Mamba-2 SSD chunked forward (gfx950).  Placeholder until the
// MFMA kernels land: reports "not supported".
#include "common.h"
#include "kernels.h"

namespace mssm {

size_t ssd_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_ssd(const SSDParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mssm
