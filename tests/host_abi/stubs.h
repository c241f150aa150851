// State shared by the host-only launcher stand-ins and the validation driver.
#pragma once
#include <cstddef>

struct StubState {
  int launches = 0;            // launchers reached since the last reset
  const char *last = "";       // name of the last launcher reached
  const void *first_out = nullptr;  // output of the first launcher after a reset
  const void *last_out = nullptr;
  int fail_next = 0;           // the next launcher returns a HIP error
  int fail_get_device = 0;     // hipGetDevice fails
  int device = 0;              // device hipGetDevice reports
  int symbol_lookups = 0;      // hipGetSymbolAddress calls
  const void *scratch_addr = nullptr;
};

extern StubState g_stub;
