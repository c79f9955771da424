// abi_stubs.hpp -- the launch log of the host stand-ins in abi_stubs.cpp.
#pragma once

#include <string>
#include <vector>

namespace stubs {
extern std::vector<std::string> g_log;  // kernel names, in launch order
extern std::string g_fail_next;         // the next launch of this kernel fails
}  // namespace stubs
