// Thread-local error text behind pkv_last_error().
#pragma once

#include <string>

namespace pkv {

std::string& last_error();

inline void clear_error() { last_error().clear(); }

inline int fail(int status, const std::string& msg) {
  last_error() = msg;
  return status;
}

}  // namespace pkv
