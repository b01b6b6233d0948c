// Error reporting shared by the C ABI translation units.
#pragma once

#include "nerf_mi355x.h"

// Records a printf-style message as this thread's last error and returns s.
nerf_status nerf_fail(nerf_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
