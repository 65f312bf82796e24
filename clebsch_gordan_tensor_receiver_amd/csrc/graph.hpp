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

// Source CSR restricted to the edges of each receiver chunk (ascending edge order per sender),
// so that a source pass over one chunk visits only edges whose per-edge data is resident.
struct SourceViews {
  std::vector<std::pair<int, int>> chunks;     // receiver ranges
  std::vector<size_t> ptr_off, edge_off;       // element offsets of each chunk's arrays in `base`
  void* base = nullptr;                        // device block holding every chunk's arrays
};

struct Graph {
  int n = 0, e = 0;
  std::vector<int32_t> row_ptr, col, recv, src_ptr, src_edge, perm;
  int max_in_degree = 0, max_out_degree = 0;
  std::map<int, DeviceGraph> dev;
  std::map<std::pair<int, long long>, SourceViews> views;  // (device, chunk cap)
  std::mutex mu;
  // Receiver chunks [i0, i1) whose edge count fits `cap` edges (a chunk holds at least one receiver).
  std::vector<std::pair<int, int>> chunks(long long cap) const;
};

cgtp_status_t build_graph(int n_nodes, int n_edges, const int32_t* recv, const int32_t* send, const int32_t* image,
                          Graph* g, std::string* err);
cgtp_status_t device_graph(Graph& g, DeviceGraph* out, std::string* err);
cgtp_status_t source_views(Graph& g, long long cap, const SourceViews** out, std::string* err);

}  // namespace cgtp
