// Thread-local text of the last failed call (internal to the library).
#pragma once

#include <string>

namespace vca {
void set_last_error(const std::string& msg);
}
