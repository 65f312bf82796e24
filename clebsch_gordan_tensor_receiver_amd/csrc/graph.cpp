// CSR construction (LunaTP section 4.1: edges of receiver i in [rowptr[i], rowptr[i+1]);
// section 4.4 and Sobek section 4.3: a source CSR for the node-feature gradient).  The device
// copy is made once per device (cgtp_graph_upload); per-chunk views of the source CSR are bounds
// into it computed on the device (cgtp_src_bounds), so no call allocates afterwards.
//
// Tie order within a receiver: (sender, image_x, image_y, image_z, input index).  A counting
// sort over receivers followed by a comparison sort inside each receiver segment; integer work
// only, so the result is exact and independent of the platform.
#include "graph.hpp"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <numeric>

namespace cgtp {

cgtp_status_t build_graph(int n_nodes, int n_edges, const int32_t* recv, const int32_t* send, const int32_t* image,
                          Graph* g, std::string* err) {
  if (n_nodes < 1 || n_edges < 0) {
    *err = "need n_nodes >= 1 and n_edges >= 0";
    return CGTP_ERR_INVALID_ARG;
  }
  if (n_edges > 0 && (!recv || !send)) {
    *err = "recv and send must be non-null";
    return CGTP_ERR_INVALID_ARG;
  }
  for (int k = 0; k < n_edges; ++k)
    if (recv[k] < 0 || recv[k] >= n_nodes || send[k] < 0 || send[k] >= n_nodes) {
      *err = "edge " + std::to_string(k) + " has a node index outside [0, n_nodes)";
      return CGTP_ERR_INVALID_ARG;
    }
  g->n = n_nodes;
  g->e = n_edges;
  g->row_ptr.assign(size_t(n_nodes) + 1, 0);
  for (int k = 0; k < n_edges; ++k) g->row_ptr[size_t(recv[k]) + 1]++;
  for (int i = 0; i < n_nodes; ++i) g->row_ptr[i + 1] += g->row_ptr[i];
  std::vector<int32_t> fill(g->row_ptr.begin(), g->row_ptr.end() - 1);
  g->perm.assign(size_t(n_edges), 0);
  for (int k = 0; k < n_edges; ++k) g->perm[size_t(fill[size_t(recv[k])]++)] = k;  // stable
  auto key_less = [&](int32_t a, int32_t b) {
    if (send[a] != send[b]) return send[a] < send[b];
    if (image) {
      for (int d = 0; d < 3; ++d)
        if (image[3 * size_t(a) + d] != image[3 * size_t(b) + d]) return image[3 * size_t(a) + d] < image[3 * size_t(b) + d];
    }
    return a < b;
  };
  g->max_in_degree = 0;
  for (int i = 0; i < n_nodes; ++i) {
    auto b = g->perm.begin() + g->row_ptr[i], e = g->perm.begin() + g->row_ptr[i + 1];
    std::sort(b, e, key_less);
    g->max_in_degree = std::max(g->max_in_degree, int(e - b));
  }
  g->col.resize(size_t(n_edges));
  g->recv.resize(size_t(n_edges));
  for (int k = 0; k < n_edges; ++k) {
    g->col[k] = send[g->perm[k]];
    g->recv[k] = recv[g->perm[k]];
  }
  g->src_ptr.assign(size_t(n_nodes) + 1, 0);
  for (int k = 0; k < n_edges; ++k) g->src_ptr[size_t(g->col[k]) + 1]++;
  for (int i = 0; i < n_nodes; ++i) g->src_ptr[i + 1] += g->src_ptr[i];
  std::vector<int32_t> sfill(g->src_ptr.begin(), g->src_ptr.end() - 1);
  g->src_edge.assign(size_t(n_edges), 0);
  for (int k = 0; k < n_edges; ++k) g->src_edge[size_t(sfill[size_t(g->col[k])]++)] = k;  // ascending k
  g->max_out_degree = 0;
  for (int i = 0; i < n_nodes; ++i) g->max_out_degree = std::max(g->max_out_degree, g->src_ptr[i + 1] - g->src_ptr[i]);
  return CGTP_OK;
}

std::vector<std::pair<int, int>> Graph::chunks(long long cap, long long rcap) const {
  std::vector<std::pair<int, int>> out;
  int i0 = 0;
  while (i0 < n) {
    int i1 = i0 + 1;
    while (i1 < n && i1 - i0 < rcap && (long long)row_ptr[i1 + 1] - row_ptr[i0] <= cap) ++i1;
    out.push_back({i0, i1});
    i0 = i1;
  }
  return out;
}

// Automatic mode orders by degree when the in-degrees are skewed: the largest exceeds twice the mean.
bool Graph::degree_order() const {
  if (order_mode == kOrderIndex) return false;
  if (order_mode == kOrderDegree) return true;
  return n > 0 && e > 0 && double(max_in_degree) > 2.0 * double(e) / double(n);
}

namespace {

// Slot order of a launch over all n nodes (LunaTP section 4.2, "task ordering": nodes by degree,
// descending, heaviest tasks first).  Slots are dealt to the 8 XCDs in contiguous ranges of
// ceil(n / 8) (the kernels' block -> XCD mapping), so each XCD keeps its own range of nodes and its
// L2 locality; inside a range the nodes are sorted by descending degree, ties by index.
std::vector<int32_t> degree_slots(const std::vector<int32_t>& ptr, int n) {
  std::vector<int32_t> ord(static_cast<size_t>(n));
  std::iota(ord.begin(), ord.end(), 0);
  const int per = (n + 7) / 8;
  for (int x = 0; x < 8; ++x) {
    const int a = std::min(n, x * per), b = std::min(n, (x + 1) * per);
    std::stable_sort(ord.begin() + a, ord.begin() + b,
                     [&](int32_t i, int32_t j) { return ptr[i + 1] - ptr[i] > ptr[j + 1] - ptr[j]; });
  }
  return ord;
}

}  // namespace

cgtp_status_t device_graph(Graph& g, DeviceGraph* out, std::string* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = "hipGetDevice failed";
    return CGTP_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g.mu);
  auto it = g.dev.find(dev);
  if (it != g.dev.end()) {
    *out = it->second;
    return CGTP_OK;
  }
  size_t n1 = size_t(g.n) + 1, ne = size_t(g.e);
  auto al = [](size_t n) { return (n * sizeof(int32_t) + 255) / 256 * 256; };
  const bool ordered = g.degree_order();
  std::vector<int32_t> rorder, sorder;
  if (ordered) {
    rorder = degree_slots(g.row_ptr, g.n);
    sorder = degree_slots(g.src_ptr, g.n);
  }
  size_t bytes = 2 * al(n1) + 3 * al(std::max<size_t>(ne, 1)) + (ordered ? 2 * al(size_t(g.n)) : 0);
  DeviceGraph d;
  hipError_t e = hipMalloc(&d.base, bytes);
  if (e != hipSuccess) {
    *err = std::string("hipMalloc(graph): ") + hipGetErrorString(e);
    return CGTP_ERR_HIP;
  }
  char* p = static_cast<char*>(d.base);
  d.row_ptr = reinterpret_cast<int32_t*>(p);
  p += al(n1);
  d.src_ptr = reinterpret_cast<int32_t*>(p);
  p += al(n1);
  d.col = reinterpret_cast<int32_t*>(p);
  p += al(std::max<size_t>(ne, 1));
  d.recv = reinterpret_cast<int32_t*>(p);
  p += al(std::max<size_t>(ne, 1));
  d.src_edge = reinterpret_cast<int32_t*>(p);
  p += al(std::max<size_t>(ne, 1));
  if (ordered) {
    d.rorder = reinterpret_cast<int32_t*>(p);
    p += al(size_t(g.n));
    d.sorder = reinterpret_cast<int32_t*>(p);
  }
  struct {
    int32_t* dst;
    const std::vector<int32_t>* src;
  } copies[] = {{d.row_ptr, &g.row_ptr}, {d.src_ptr, &g.src_ptr}, {d.col, &g.col}, {d.recv, &g.recv},
                {d.src_edge, &g.src_edge}, {d.rorder, &rorder}, {d.sorder, &sorder}};
  for (auto& c : copies) {
    if (c.src->empty()) continue;
    e = hipMemcpy(c.dst, c.src->data(), c.src->size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      *err = std::string("hipMemcpy(graph): ") + hipGetErrorString(e);
      (void)hipFree(d.base);  // already failing: release and report the first error
      return CGTP_ERR_HIP;
    }
  }
  g.dev[dev] = d;
  *out = d;
  return CGTP_OK;
}

cgtp_status_t resident_graph(Graph& g, DeviceGraph* out, std::string* err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = "hipGetDevice failed";
    return CGTP_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g.mu);
  auto it = g.dev.find(dev);
  if (it == g.dev.end()) {
    *err = "the graph is not on device " + std::to_string(dev) + ": call cgtp_graph_upload first";
    return CGTP_ERR_INVALID_ARG;
  }
  *out = it->second;
  return CGTP_OK;
}

}  // namespace cgtp
