// abi_internal.h -- host helpers shared by the sources that implement moe.h.
#pragma once

#include "moe.h"

namespace moe {

// Sets the message moe_last_error() returns on this thread (printf format) and
// returns `s`.
moe_status set_error(moe_status s, const char *fmt, ...);

}  // namespace moe
