// Host stand-in for <hip/hip_runtime.h> used by the CPU emulation of the
// device code (tests only).
#pragma once
#include "../simt.hpp"
