// Host-side helpers shared by the library's C ABI files.
#pragma once

#include <string>

#include "../../include/lmstep.h"

namespace lm {
// Records msg as this thread's lm_last_error() text and returns st.
lm_status set_error(lm_status st, const std::string& msg);
}  // namespace lm
