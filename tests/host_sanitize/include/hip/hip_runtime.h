/* Test-only stand-in; see hip_runtime_api.h beside it. */
#include "hip_runtime_api.h"
