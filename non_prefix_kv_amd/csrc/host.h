// Host-side helpers shared by the runtime sources of libcacheblend.so.
#pragma once

#include "../../include/cacheblend.h"

namespace cb {

// Records the message cb_last_error() returns on this thread; returns st.
cb_status set_error(cb_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

enum class MemKind { Device, Pinned, Other };
// Where a pointer lives, from the HIP runtime's pointer attributes.
MemKind mem_kind(const void* p);

}  // namespace cb
