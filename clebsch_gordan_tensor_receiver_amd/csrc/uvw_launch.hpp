// Launch sequences of the fully connected (uvw) streamed convolution.
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>

#include "cgtp.h"
#include "graph.hpp"
#include "plan.hpp"

namespace cgtp {

size_t uvw_workspace(const Plan& p, const Graph& g, cgtp_op_t op);
cgtp_status_t uvw_forward(Plan& p, Graph& G, const DeviceGraph& d, const void* x, const void* pos, const void* shift,
                          const void* phi, const void* A, void* out, void* workspace, hipStream_t s,
                          std::string* err);
cgtp_status_t uvw_backward(Plan& p, Graph& G, const DeviceGraph& d, const SourceViews* views, const void* x,
                           const void* pos, const void* shift, const void* phi, const void* A, const void* gout,
                           void* grad_x, void* grad_pos, void* grad_edge_vec, void* grad_phi, void* grad_A,
                           void* workspace, hipStream_t s, std::string* err);

}  // namespace cgtp
