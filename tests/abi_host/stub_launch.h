// stub_launch.h -- what the stand-in launchers of stub_launch.cpp record.
#pragma once

#include "fa_launch.h"

namespace stub {
struct Last {
  const char* what;  // launcher reached, or nullptr
  int a, b, c, d, e, f;
};
extern Last last;
}  // namespace stub
