// Host-side launchers of the HIP kernels, for the C ABI layer: one header
// per kernel source, so that each kernel compiles from its own declarations
// only.
#pragma once

#include "launch_append.h"
#include "launch_decode.h"
#include "launch_prefill.h"
