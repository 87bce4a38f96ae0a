// Library-internal entry points shared between the host sources (not part
// of the C ABI in include/fd.h).
#pragma once

#include <cstdint>

#include "../../include/fd.h"

namespace fd {

// fd_step with `ws` (ws_bytes bytes, 256-byte aligned, device memory of the
// ctx's GPU) in place of the ctx's fd_init workspace.  Clears the plan's
// split-counter region first; creates no events.  FD_E_UNSUPPORTED for
// FD_EXEC_WALK profiles and for profiles whose workspace exceeds ws_bytes.
fd_status step_on_workspace(fd_ctx* c, void* ws, uint64_t ws_bytes, const void* x_in, void* y_out,
                            void* depth_out, void* stream);

// Device the ctx was created on.
int ctx_device(const fd_ctx* c);

}  // namespace fd
