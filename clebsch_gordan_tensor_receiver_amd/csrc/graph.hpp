// Receiver and source CSR of an edge list, on the host and (once per device) on the GPU.
#pragma once

#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "cgtp.h"

namespace cgtp {

struct DeviceGraph {
  void* base = nullptr;
  int32_t *row_ptr = nullptr, *col = nullptr, *recv = nullptr, *src_ptr = nullptr, *src_edge = nullptr;
};

struct Graph {
  int n = 0, e = 0;
  std::vector<int32_t> row_ptr, col, recv, src_ptr, src_edge, perm;
  int max_in_degree = 0, max_out_degree = 0;
  std::map<int, DeviceGraph> dev;
  std::mutex mu;
  // Receiver chunks [i0, i1) whose edge count fits `cap` edges (a chunk holds at least one receiver).
  std::vector<std::pair<int, int>> chunks(long long cap) const;
};

cgtp_status_t build_graph(int n_nodes, int n_edges, const int32_t* recv, const int32_t* send, const int32_t* image,
                          Graph* g, std::string* err);
cgtp_status_t device_graph(Graph& g, DeviceGraph* out, std::string* err);

}  // namespace cgtp
