// The channelwise forward with its workspace and chunk budget given explicitly (api.cpp), for the
// allocation-free entry point (noalloc.hip): the G rows of each receiver chunk go to `scratch`, the
// chunks are cut so that they fit `scratch_bytes`, the graph must already be on the device and
// the plan's forward kernels loaded there.  Nothing is uploaded, compiled or loaded.
#pragma once

#include <cstddef>

#include "cgtp.h"

namespace cgtp {
cgtp_status_t forward_in_scratch(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                 const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                 void* scratch, size_t scratch_bytes, void* stream);
}  // namespace cgtp
