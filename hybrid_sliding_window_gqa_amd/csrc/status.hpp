// Error reporting shared by the library's entry points: the message for the
// last failure on the calling thread, returned by ha_last_error().
#pragma once

#include "../../include/hybrid_attn.h"

namespace ha {

// Records a printf-style message and returns st.
ha_status set_error(ha_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the message and returns HA_OK.
ha_status clear_error();

}  // namespace ha
