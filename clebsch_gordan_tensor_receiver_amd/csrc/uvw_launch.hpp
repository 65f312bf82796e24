// Launch sequences of the fully connected (uvw) streamed convolution.
#pragma once

#include <hip/hip_runtime_api.h>

#include <string>

#include "cgtp.h"
#include "graph.hpp"
#include "plan.hpp"

namespace cgtp {

size_t uvw_workspace(const Plan& p, const Graph& g, cgtp_op_t op);
// Bytes of the receiver state S of every node (node-major, the per-node layout of the state
// kernel's output).
size_t uvw_state_bytes(const Plan& p, const Graph& g);
// `state` (nullable): the forward writes S of every node there instead of into the workspace.
cgtp_status_t uvw_forward(Plan& p, Graph& G, const DeviceGraph& d, const void* x, const void* pos, const void* shift,
                          const void* phi, const void* A, void* out, void* workspace, hipStream_t s,
                          std::string* err, void* state = nullptr);
// `state` (nullable): S kept by the forward; the backward then reads it instead of recomputing it.
cgtp_status_t uvw_backward(Plan& p, Graph& G, const DeviceGraph& d, const void* x,
                           const void* pos, const void* shift, const void* phi, const void* A, const void* gout,
                           void* grad_x, void* grad_pos, void* grad_edge_vec, void* grad_phi, void* grad_A,
                           void* workspace, hipStream_t s, std::string* err, const void* state = nullptr);

// Double backward (Sobek section 3.3 and Eqs. 37-39) by linearity: every second-order output is a
// sum of first-order passes with one operand replaced by its direction.  Directions nullable.
cgtp_status_t uvw_double_backward(Plan& p, Graph& G, const DeviceGraph& d, const void* x, const void* pos,
                                  const void* shift, const void* phi, const void* A, const void* gout,
                                  const void* v_x, const void* v_pos, const void* v_edge_vec, const void* v_phi,
                                  const void* v_A, void* gg_x, void* gg_pos, void* gg_edge_vec, void* gg_phi,
                                  void* gg_A, void* gg_grad_out, void* workspace, hipStream_t s, std::string* err,
                                  void* phibar_out = nullptr);

}  // namespace cgtp
