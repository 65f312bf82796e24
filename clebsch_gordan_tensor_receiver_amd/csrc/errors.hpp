// Status reporting shared by the library's translation units: set_error records the message that
// cgtp_last_error() returns to the calling thread and passes the status through.
#pragma once

#include <string>

#include "cgtp.h"

namespace cgtp {
cgtp_status_t set_error(cgtp_status_t status, const std::string& message);
}  // namespace cgtp
