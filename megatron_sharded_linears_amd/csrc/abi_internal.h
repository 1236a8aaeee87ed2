// Internal entry points of the C ABI layer (abi.cpp) for other translation
// units of the library: validation and dispatch of one linear, and the
// scratch its automatic plan needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_shard.h"

namespace tpabi {

// Validate and run the linear `c` describes (what tp_linear_ex does).
int linear_call(const tp_linear_call& c, hipStream_t s);

// Host only, no HIP call: validate `c` as linear_call would (its workspace
// fields ignored) and report the scratch its kernel plan needs when given a
// workspace of tp_workspace_bytes(): fp32 floats and arrival counters (both
// zero when K stays within one workgroup).
int linear_scratch_need(const tp_linear_call& c, int64_t* floats, int64_t* counters);

}  // namespace tpabi
