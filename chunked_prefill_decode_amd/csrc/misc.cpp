// Error text and version of libsarathi_attn.
#include <string>

#include "common.h"

namespace sa {
std::string& last_error() {
  thread_local std::string text;
  return text;
}
}  // namespace sa

extern "C" {
const char* sa_last_error(void) { return sa::last_error().c_str(); }
const char* sa_version(void) { return "sarathi_attn 0.1 gfx950"; }
}
