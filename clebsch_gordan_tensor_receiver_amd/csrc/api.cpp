// The extern "C" surface declared in include/cgtp.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "cgtp.h"
#include "errors.hpp"
#include "forward.hpp"
#include "graph.hpp"
#include "kernels.hpp"
#include "plan.hpp"
#include "uvw_launch.hpp"

struct cgtp_plan_s {
  cgtp::Plan p;
};
struct cgtp_graph_s {
  cgtp::Graph g;
};

namespace {

thread_local std::string g_last_error;

cgtp_status_t fail(cgtp_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

cgtp_status_t ok() {
  g_last_error.clear();
  return CGTP_OK;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Edges of G rows that fit in `budget` bytes (at least the largest in-degree).
long long g_chunk_edges(const cgtp::Plan& p, const cgtp::Graph& g, size_t budget) {
  long long row = (long long)p.g_stride * (long long)p.elem();
  long long cap = std::max<long long>(1, (long long)(budget / size_t(row)));
  return std::max<long long>(cap, g.max_in_degree);
}

long long max_chunk_edges(const cgtp::Graph& g, const std::vector<std::pair<int, int>>& ch) {
  long long m = 0;
  for (auto& c : ch) m = std::max<long long>(m, g.row_ptr[c.second] - g.row_ptr[c.first]);
  return m;
}

// Channelwise forward workspace: the G rows of the largest receiver chunk under `budget`.
size_t forward_rows_bytes(const cgtp::Plan& p, const cgtp::Graph& g, size_t budget) {
  auto ch = g.chunks(g_chunk_edges(p, g, budget));
  return align256(size_t(max_chunk_edges(g, ch)) * size_t(p.g_stride) * p.elem());
}

// Launch geometry shared with the generated kernels (codegen.cpp).
constexpr int kSrcSplit = 2;    // waves per sender in the source backward
constexpr int kRecvGroup = 4;   // receivers (one wave each) per workgroup in the receiver backward

// Workspace plan of a backward or double-backward call.
struct BwdLayout {
  long long cap = 0;            // edges per receiver chunk
  long long rcap = 0;           // receivers per chunk (bounds the A-bar partial slots)
  std::vector<std::pair<int, int>> chunks;
  int ntask_r = 0, ntask_s = 0, V = 0, row = 0;
  int nslot = 0;                // A-bar partial slots (max over chunks)
  long long emax = 0;           // edges of the largest chunk (stride of the edge partials)
  size_t g_off = 0, ep_off = 0, ap_off = 0, gev_off = 0, sb_off = 0, total = 0;
};

// Receivers per XCD and receiver groups per XCD of a chunk; the groups are the A-bar slots.
void chunk_geometry(int nrec, int* per, int* nch) {
  *per = (nrec + 7) / 8;
  *nch = (*per + kRecvGroup - 1) / kRecvGroup;
}

// Shared by the backward (grow = G + Y values per edge) and the double backward (grow = G and its
// tangent).  The scratch budget covers the per-edge rows, the edge partials and the A-bar slots
// (K x N_w values each, one per workgroup of 4 receivers).  It is split between the two in the
// ratio of their cost per receiver at the graph's mean in-degree: the slot share caps the
// receivers per chunk, the row share the edges per chunk, so that neither grows with the other
// (a low-degree graph has many receivers per edge).  Beyond the budget the workspace holds E x 3
// edge-vector values and, with several chunks, the begin/end bounds of each sender's source-CSR
// run (2 N int32).
BwdLayout chunked_layout(const cgtp::Plan& p, const cgtp::Graph& g, int grow, int row, int ntask_r) {
  BwdLayout L;
  L.ntask_r = ntask_r;
  L.ntask_s = int(cgtp::source_tasks(p).size());
  L.V = 0;
  L.row = row;
  const size_t slot_bytes = size_t(p.K) * size_t(p.n_w) * p.elem();
  long long row_bytes = (long long)(grow + L.row) * (long long)p.elem();
  const double deg = g.n > 0 ? double(g.e) / double(g.n) : 1.0;
  const double per_recv_slots = double(slot_bytes) / kRecvGroup, per_recv_rows = deg * double(row_bytes);
  const double frac = std::min(7.0 / 8.0, std::max(1.0 / 16.0, per_recv_slots / (per_recv_slots + per_recv_rows)));
  const size_t slot_share = size_t(frac * double(p.scratch_budget));
  const long long nch_max = std::max<long long>(1, (long long)(slot_share / slot_bytes) / 8);
  L.rcap = 8LL * kRecvGroup * nch_max;
  const size_t slot_area = size_t(8 * nch_max) * slot_bytes;
  const size_t rest = p.scratch_budget > slot_area ? p.scratch_budget - slot_area : 0;
  L.cap = std::max<long long>(std::max<long long>(1, (long long)(rest / size_t(row_bytes))), g.max_in_degree);
  L.chunks = g.chunks(L.cap, L.rcap);
  long long emax = std::max<long long>(1, max_chunk_edges(g, L.chunks));
  L.emax = emax;
  for (auto& c : L.chunks) {
    int per, nch;
    chunk_geometry(c.second - c.first, &per, &nch);
    L.nslot = std::max(L.nslot, 8 * nch);
  }
  size_t off = 0;
  L.g_off = off;
  off += align256(size_t(emax) * size_t(grow) * p.elem());
  L.ep_off = off;
  off += align256(size_t((emax + 63) / 64 * 64) * size_t(L.row) * p.elem());  // tiles of 64 edges
  L.ap_off = off;
  off += align256(size_t(L.nslot) * slot_bytes);
  L.gev_off = off;
  off += align256(size_t(std::max(g.e, 1)) * 3 * p.elem());
  L.sb_off = off;
  if (L.chunks.size() > 1) off += align256(2 * size_t(g.n) * sizeof(int32_t));
  L.total = off;
  return L;
}

BwdLayout bwd_layout(const cgtp::Plan& p, const cgtp::Graph& g) {
  return chunked_layout(p, g, cgtp::bwd_row_stride(p), cgtp::recv_partial_row(p),
                        int(cgtp::recv_backward_tasks(p).size()));
}

// Double backward: G and Gdot rows (2 g_stride per edge), the edge partials of the receiver pass,
// A-bar-dot slots, an edge-vector buffer.
BwdLayout dbl_layout(const cgtp::Plan& p, const cgtp::Graph& g) {
  return chunked_layout(p, g, 2 * p.g_stride, cgtp::dbl_partial_row(p), int(cgtp::dbl_recv_tasks(p).size()));
}

// Begin/end bounds of every sender's out-edges inside receiver chunk c, for the source passes.
// One chunk: the whole source CSR (src_ptr and src_ptr + 1).  Several: computed on the device
// into the workspace (cgtp_src_bounds), in stream order before the chunk's source pass.
cgtp_status_t source_bounds(cgtp::Plan& p, const char* fam, const cgtp::Graph& G, const cgtp::DeviceGraph& d,
                            const BwdLayout& L, size_t c, char* ws, hipStream_t s, void** beg, void** end,
                            std::string* err) {
  if (L.chunks.size() == 1) {
    *beg = d.src_ptr;
    *end = d.src_ptr + 1;
    return CGTP_OK;
  }
  hipFunction_t kb;
  cgtp_status_t st = cgtp::get_kernel(p, fam, "cgtp_src_bounds", &kb, err);
  if (st != CGTP_OK) return st;
  int32_t* b = reinterpret_cast<int32_t*>(ws + L.sb_off);
  *beg = b;
  *end = b + G.n;
  int n = G.n, e0 = G.row_ptr[L.chunks[c].first], e1 = G.row_ptr[L.chunks[c].second];
  void* a[] = {(void*)&d.src_ptr, (void*)&d.src_edge, &n, &e0, &e1, beg, end};
  return cgtp::launch(kb, unsigned((n + 255) / 256), 256, 0, s, a, err);
}

// The plan with 2K radial values of the third-order passes (created on first use).
cgtp_status_t tri_plan(cgtp::Plan& p, cgtp::Plan** out, std::string* err) {
  std::lock_guard<std::mutex> lock(p.mu);
  if (!p.tri) {
    if (2 * p.K > 64) {
      *err = "the third-order passes need 2K <= 64 radial values";
      return CGTP_ERR_UNSUPPORTED;
    }
    std::unique_ptr<cgtp::Plan> t(new cgtp::Plan());
    cgtp_status_t st = cgtp::build_plan(p.irreps_in_s.c_str(), p.irreps_sh_s.c_str(), p.irreps_out_s.c_str(), p.mode,
                                        p.dtype, 2 * p.K, t.get(), err);
    if (st != CGTP_OK) return st;
    t->scratch_budget = p.scratch_budget;
    p.tri = std::move(t);
  }
  p.tri->scratch_budget = p.scratch_budget;
  *out = p.tri.get();
  return CGTP_OK;
}

// The plan's twin without a radial basis (created on first use): the fully connected double
// backward of a plan with one runs on it, phi and phi-dot materialised per edge.
cgtp_status_t plain_plan(cgtp::Plan& p, cgtp::Plan** out, std::string* err) {
  std::lock_guard<std::mutex> lock(p.mu);
  if (!p.plain) {
    std::unique_ptr<cgtp::Plan> t(new cgtp::Plan());
    cgtp_status_t st = cgtp::build_plan(p.irreps_in_s.c_str(), p.irreps_sh_s.c_str(), p.irreps_out_s.c_str(), p.mode,
                                        p.dtype, p.K, t.get(), err);
    if (st != CGTP_OK) return st;
    p.plain = std::move(t);
  }
  p.plain->scratch_budget = p.scratch_budget;
  *out = p.plain.get();
  return CGTP_OK;
}

// Workspace of the fully connected double backward with a radial basis: phi, phi-dot, the
// gradient in phi and the first-order phi-bar (E x K each), e-bar-dot (E x 3), then the workspace
// of the double backward on the plain twin.
struct RadialDblLayout {
  size_t phi_off = 0, vphi_off = 0, gphi_off = 0, pb_off = 0, gev_off = 0, inner_off = 0, total = 0;
};
RadialDblLayout radial_dbl_layout(const cgtp::Plan& p, const cgtp::Plan& pp, const cgtp::Graph& G) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  RadialDblLayout L;
  const size_t ek = al(size_t(std::max(G.e, 1)) * p.K * p.elem());
  L.phi_off = 0;
  L.vphi_off = ek;
  L.gphi_off = 2 * ek;
  L.pb_off = 3 * ek;
  L.gev_off = 4 * ek;
  L.inner_off = L.gev_off + al(size_t(std::max(G.e, 1)) * 3 * p.elem());
  L.total = L.inner_off + cgtp::uvw_workspace(pp, G, CGTP_OP_DOUBLE_BACKWARD);
  return L;
}

// Workspace of the third-order passes (on the 2K plan tp): per edge of a receiver chunk the rows of
// one edge operand (Y, v_Y or q_Y: the terms run grouped by it) and the packed radial factors
// (2K); the receiver pass's partials and A-bar slots; beyond the budget the packed A factors
// (2K x N_w) and the chunked source bounds.  Every pass adds its results into the outputs.
struct TriLayout {
  BwdLayout L;
  size_t gy_off[3] = {0, 0, 0}, pk_off = 0, ak_off = 0, total = 0;
};

TriLayout tri_layout(const cgtp::Plan& p, const cgtp::Plan& tp, const cgtp::Graph& g) {
  TriLayout T;
  const int rs = cgtp::bwd_row_stride(tp), K2 = tp.K;
  const int grow = rs + K2;   // the rows of one edge operand at a time, and the packed radial factors
  // The receiver passes run on the 2K plan (stacked factors) or on the plan itself (one factor):
  // partial rows for the wider of the two; the A-bar slots are sized by the 2K plan.
  const int row = std::max(cgtp::recv_partial_row(tp), cgtp::recv_partial_row(p));
  T.L = chunked_layout(tp, g, grow, row, int(cgtp::recv_backward_tasks(tp).size()));
  const size_t em = size_t(T.L.emax), el = tp.elem();
  size_t off = T.L.g_off;
  T.gy_off[0] = T.gy_off[1] = T.gy_off[2] = off;
  off += em * size_t(rs) * el;
  T.pk_off = off;
  off = T.L.total;
  T.ak_off = off;
  off += align256(size_t(K2) * size_t(tp.n_w) * el);
  T.total = off;
  return T;
}

// Feature blocks that no path reaches (output side) or leaves (input side) are not written by
// the kernels; zero the whole tensor first when such a block exists.
cgtp_status_t zero_unreached(cgtp::Plan& p, void* buf, int n, bool out_side, hipStream_t s, std::string* err,
                             bool loaded_only = false) {
  const auto& blocks = out_side ? p.out : p.in;
  const auto& by = out_side ? p.by_out : p.by_in;
  bool any = false;
  for (size_t k = 0; k < blocks.size(); ++k) any = any || by[k].empty();
  if (!any) return CGTP_OK;
  const char* fam = p.mode == CGTP_CHANNELWISE ? "fwd" : "uvw_fwd";
  hipFunction_t kz;
  cgtp_status_t st = cgtp::get_kernel(p, fam, "cgtp_fill_zero", &kz, err, loaded_only);
  if (st != CGTP_OK) return st;
  long long cnt = (long long)n * (out_side ? p.c_out : p.c_in);
  void* a[] = {&buf, &cnt};
  return cgtp::launch(kz, unsigned((cnt + 255) / 256), 256, 0, s, a, err);
}

}  // namespace

namespace cgtp {
cgtp_status_t set_error(cgtp_status_t status, const std::string& message) {
  g_last_error = message;
  return status;
}
}  // namespace cgtp

extern "C" {

const char* cgtp_error_string(cgtp_status_t s) {
  switch (s) {
    case CGTP_OK: return "ok";
    case CGTP_ERR_INVALID_ARG: return "invalid argument";
    case CGTP_ERR_UNSUPPORTED: return "unsupported";
    case CGTP_ERR_WORKSPACE: return "workspace too small";
    case CGTP_ERR_DEGENERATE_EDGE: return "zero-length edge";
    case CGTP_ERR_HIP: return "HIP runtime error";
    case CGTP_ERR_COMPILE: return "kernel compilation failed";
  }
  return "unknown status";
}

const char* cgtp_last_error(void) { return g_last_error.c_str(); }

cgtp_status_t cgtp_plan_create(const char* irreps_in, const char* irreps_sh, const char* irreps_out, cgtp_mode_t mode,
                               cgtp_dtype_t dtype, int num_radial, cgtp_plan_t* out) {
  if (!out) return fail(CGTP_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  cgtp_plan_s* h = new (std::nothrow) cgtp_plan_s();
  if (!h) return fail(CGTP_ERR_INVALID_ARG, "out of host memory");
  std::string err;
  cgtp_status_t st = cgtp::build_plan(irreps_in, irreps_sh, irreps_out, mode, dtype, num_radial, &h->p, &err);
  if (st != CGTP_OK) {
    delete h;
    return fail(st, err);
  }
  *out = h;
  return ok();
}

cgtp_status_t cgtp_plan_destroy(cgtp_plan_t plan) {
  delete plan;
  return ok();
}

cgtp_status_t cgtp_plan_info(cgtp_plan_t plan, cgtp_plan_info_t* out) {
  if (!plan || !out) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  const cgtp::Plan& p = plan->p;
  out->n_paths = int(p.paths.size());
  out->n_weights = p.n_w;
  out->c_in = p.c_in;
  out->c_out = p.c_out;
  out->sh_dim = p.sh_dim;
  out->lmax_sh = p.lmax;
  out->num_radial = p.K;
  out->mode = int(p.mode);
  out->dtype = int(p.dtype);
  out->n_in_blocks = int(p.in.size());
  out->n_out_blocks = int(p.out.size());
  out->cg_nnz = p.cg_nnz;
  out->g_nnz = p.g_width;
  return ok();
}

cgtp_status_t cgtp_plan_path(cgtp_plan_t plan, int path, int32_t* desc) {
  if (!plan || !desc) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  if (path < 0 || path >= int(plan->p.paths.size())) return fail(CGTP_ERR_INVALID_ARG, "path out of range");
  const cgtp::Path& P = plan->p.paths[path];
  int32_t v[9] = {P.i_in, P.i_sh, P.i_out, P.l1, P.l2, P.l3, P.w_off, P.n_w, int32_t(P.terms.size())};
  std::memcpy(desc, v, sizeof v);
  return ok();
}

cgtp_status_t cgtp_plan_cg_table(cgtp_plan_t plan, int path, int32_t* m123, double* val, int capacity, int* nnz) {
  if (!plan || !nnz) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  if (path < 0 || path >= int(plan->p.paths.size())) return fail(CGTP_ERR_INVALID_ARG, "path out of range");
  const cgtp::Path& P = plan->p.paths[path];
  *nnz = int(P.terms.size());
  for (int k = 0; k < std::min(capacity, *nnz); ++k) {
    if (m123) {
      m123[3 * k] = P.terms[k].m1;
      m123[3 * k + 1] = P.terms[k].m2;
      m123[3 * k + 2] = P.terms[k].m3;
    }
    if (val) val[k] = P.terms[k].c;
  }
  return ok();
}

cgtp_status_t cgtp_plan_set_scratch_budget(cgtp_plan_t plan, size_t bytes) {
  if (!plan || bytes < 4096) return fail(CGTP_ERR_INVALID_ARG, "budget must be at least 4096 bytes");
  plan->p.scratch_budget = bytes;
  return ok();
}

cgtp_status_t cgtp_plan_set_radial(cgtp_plan_t plan, int kind, double r_cut) {
  if (!plan) return fail(CGTP_ERR_INVALID_ARG, "null plan");
  if (kind < 0 || kind > 2) return fail(CGTP_ERR_INVALID_ARG, "radial kind must be 0, 1 or 2");
  if (kind != 0 && !(r_cut > 0.0)) return fail(CGTP_ERR_INVALID_ARG, "cutoff radius must be positive");
  if (kind == 2 && plan->p.K < 2) return fail(CGTP_ERR_INVALID_ARG, "the Gaussian basis needs K >= 2");
  cgtp::Plan& p = plan->p;
  std::lock_guard<std::mutex> lock(p.mu);
  if (!p.kernels->families.empty())
    return fail(CGTP_ERR_UNSUPPORTED, "set the radial basis before the plan's kernels are compiled");
  p.radial = kind;
  p.r_cut = kind ? r_cut : 0.0;
  p.phi_off = p.g_width;
  p.g_stride = (p.g_width + (kind ? p.K : 0) + 3) / 4 * 4;
  return ok();
}

cgtp_status_t cgtp_plan_compile(cgtp_plan_t plan, int ops) {
  if (!plan) return fail(CGTP_ERR_INVALID_ARG, "null plan");
  std::string err;
  std::vector<std::string> fams;
  if (plan->p.mode == CGTP_CHANNELWISE) {
    if (ops & (1 << CGTP_OP_FORWARD)) {
      fams.push_back("fwd");
      fams.push_back("fwds");
    }
    if (ops & (1 << CGTP_OP_BACKWARD)) fams.push_back("bwd");
    // Forward and backward together: also the forward that keeps its edge rows for the backward.
    if ((ops & (1 << CGTP_OP_FORWARD)) && (ops & (1 << CGTP_OP_BACKWARD))) fams.push_back("fwdk");
    if (ops & (1 << CGTP_OP_DOUBLE_BACKWARD)) fams.push_back("dbl");
    if (ops & (1 << CGTP_OP_TRIPLE_BACKWARD)) {
      cgtp::Plan* tp = nullptr;
      cgtp_status_t st = tri_plan(plan->p, &tp, &err);
      if (st == CGTP_OK) st = cgtp::compile_family(*tp, "tri", &err);
      if (st == CGTP_OK) st = cgtp::compile_family(plan->p, "tri1", &err);
      if (st != CGTP_OK) return fail(st, err);
    }
  } else {
    if (ops & (1 << CGTP_OP_TRIPLE_BACKWARD))
      return fail(CGTP_ERR_UNSUPPORTED, "the triple backward is channelwise only");
    if (ops & (1 << CGTP_OP_FORWARD)) fams.push_back("uvw_fwd");
    if (ops & (1 << CGTP_OP_BACKWARD)) fams.push_back("uvw_bwd");
    if (ops & (1 << CGTP_OP_DOUBLE_BACKWARD)) {
      if (plan->p.radial) {
        cgtp::Plan* pp = nullptr;
        cgtp_status_t st = plain_plan(plan->p, &pp, &err);
        if (st == CGTP_OK) st = cgtp::compile_family(*pp, "uvw_dbl", &err);
        if (st != CGTP_OK) return fail(st, err);
        fams.push_back("uvw_rdbl");
      } else {
        fams.push_back("uvw_dbl");
      }
    }
  }
  if (ops & (1 << CGTP_OP_FORWARD)) fams.push_back("layout");  // boundary layout conversion
  for (auto& f : fams) {
    cgtp_status_t st = cgtp::compile_family(plan->p, f, &err);
    if (st != CGTP_OK) return fail(st, err);
  }
  return ok();
}

cgtp_status_t cgtp_graph_build(int n_nodes, int n_edges, const int32_t* recv, const int32_t* send,
                               const int32_t* image, int32_t* perm_out, cgtp_graph_t* out) {
  if (!out) return fail(CGTP_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  cgtp_graph_s* h = new (std::nothrow) cgtp_graph_s();
  if (!h) return fail(CGTP_ERR_INVALID_ARG, "out of host memory");
  std::string err;
  cgtp_status_t st = cgtp::build_graph(n_nodes, n_edges, recv, send, image, &h->g, &err);
  if (st != CGTP_OK) {
    delete h;
    return fail(st, err);
  }
  if (perm_out && n_edges > 0) std::memcpy(perm_out, h->g.perm.data(), sizeof(int32_t) * size_t(n_edges));
  *out = h;
  return ok();
}

cgtp_status_t cgtp_graph_export(cgtp_graph_t g, int32_t* row_ptr, int32_t* col, int32_t* src_ptr, int32_t* src_edge) {
  if (!g) return fail(CGTP_ERR_INVALID_ARG, "null graph");
  const cgtp::Graph& G = g->g;
  if (row_ptr) std::memcpy(row_ptr, G.row_ptr.data(), sizeof(int32_t) * G.row_ptr.size());
  if (src_ptr) std::memcpy(src_ptr, G.src_ptr.data(), sizeof(int32_t) * G.src_ptr.size());
  if (col && G.e) std::memcpy(col, G.col.data(), sizeof(int32_t) * G.col.size());
  if (src_edge && G.e) std::memcpy(src_edge, G.src_edge.data(), sizeof(int32_t) * G.src_edge.size());
  return ok();
}

cgtp_status_t cgtp_graph_dims(cgtp_graph_t g, int* n_nodes, int* n_edges) {
  if (!g) return fail(CGTP_ERR_INVALID_ARG, "null graph");
  if (n_nodes) *n_nodes = g->g.n;
  if (n_edges) *n_edges = g->g.e;
  return ok();
}

cgtp_status_t cgtp_graph_set_order(cgtp_graph_t g, int mode) {
  if (!g) return fail(CGTP_ERR_INVALID_ARG, "null graph");
  if (mode < 0 || mode > 2) return fail(CGTP_ERR_INVALID_ARG, "order mode must be 0, 1 or 2");
  std::lock_guard<std::mutex> lock(g->g.mu);
  if (!g->g.dev.empty()) return fail(CGTP_ERR_UNSUPPORTED, "set the order before the graph is uploaded");
  g->g.order_mode = mode;
  return ok();
}

cgtp_status_t cgtp_graph_upload(cgtp_graph_t g) {
  if (!g) return fail(CGTP_ERR_INVALID_ARG, "null graph");
  cgtp::DeviceGraph d;
  std::string err;
  cgtp_status_t st = cgtp::device_graph(g->g, &d, &err);
  return st == CGTP_OK ? ok() : fail(st, err);
}

cgtp_status_t cgtp_graph_destroy(cgtp_graph_t g) {
  if (!g) return ok();
  // Best-effort release on every device the graph was uploaded to (errors cannot be reported
  // from a destructor-like call and do not leak host state).
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g->g.dev) {
    (void)hipSetDevice(kv.first);
    (void)hipFree(kv.second.base);
  }
  (void)hipSetDevice(cur);
  delete g;
  return ok();
}

cgtp_status_t cgtp_workspace_size(cgtp_plan_t plan, cgtp_graph_t g, cgtp_op_t op, size_t* bytes) {
  if (!plan || !g || !bytes) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  const cgtp::Plan& p = plan->p;
  const cgtp::Graph& G = g->g;
  size_t need = 0;
  if (p.mode == CGTP_FULLY_CONNECTED) {
    if (op == CGTP_OP_TRIPLE_BACKWARD) return fail(CGTP_ERR_UNSUPPORTED, "the triple backward is channelwise only");
    if (op == CGTP_OP_DOUBLE_BACKWARD && p.radial) {
      cgtp::Plan* pp = nullptr;
      std::string err;
      cgtp_status_t st = plain_plan(plan->p, &pp, &err);
      if (st != CGTP_OK) return fail(st, err);
      *bytes = std::max<size_t>(radial_dbl_layout(p, *pp, G).total, 256);
      return ok();
    }
    *bytes = std::max<size_t>(cgtp::uvw_workspace(p, G, op), 256);
    return ok();
  }
  if (op == CGTP_OP_TRIPLE_BACKWARD) {
    cgtp::Plan* tp = nullptr;
    std::string err;
    cgtp_status_t st = tri_plan(plan->p, &tp, &err);
    if (st != CGTP_OK) return fail(st, err);
    need = tri_layout(plan->p, *tp, G).total;
  } else if (op == CGTP_OP_FORWARD) {
    need = forward_rows_bytes(p, G, p.scratch_budget);
  } else if (op == CGTP_OP_BACKWARD) {
    need = bwd_layout(p, G).total;
  } else {
    need = dbl_layout(p, G).total;
  }
  *bytes = std::max<size_t>(need, 256);
  return ok();
}

// `budget`: bytes of G rows per receiver chunk (the plan's scratch budget, or the static scratch of
// the allocation-free entry point).  `no_alloc`: the graph must already be on the device and the
// kernels loaded there; nothing is uploaded, compiled or loaded (no device allocation).
static cgtp_status_t conv_forward_impl(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                       const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                       void* workspace, size_t ws_bytes, void* stream, void* state, size_t budget,
                                       bool no_alloc) {
  if (!plan || !g) return fail(CGTP_ERR_INVALID_ARG, "null plan or graph");
  if (!x || !pos || !A || !out) return fail(CGTP_ERR_INVALID_ARG, "null tensor argument");
  if (schedule != CGTP_STREAMED && schedule != CGTP_CONVENTIONAL) return fail(CGTP_ERR_INVALID_ARG, "bad schedule");
  cgtp::Plan& p = plan->p;
  if ((phi == nullptr) != (p.radial != 0))
    return fail(CGTP_ERR_INVALID_ARG, p.radial ? "phi must be NULL: the plan computes the radial basis"
                                               : "null phi (the plan has no radial basis of its own)");
  cgtp::Graph& G = g->g;
  size_t need = 0;
  if (no_alloc)
    need = p.mode == CGTP_CHANNELWISE ? forward_rows_bytes(p, G, budget) : 0;
  else
    cgtp_workspace_size(plan, g, CGTP_OP_FORWARD, &need);
  if (ws_bytes < need || (!workspace && need > 0))
    return fail(CGTP_ERR_WORKSPACE, "workspace too small: " + std::to_string(need) + " bytes needed, " +
                                        std::to_string(ws_bytes) + " given");
  std::string err;
  cgtp::DeviceGraph d;
  cgtp_status_t st = no_alloc ? cgtp::resident_graph(G, &d, &err) : cgtp::device_graph(G, &d, &err);
  if (st != CGTP_OK) return fail(st, err);
  hipStream_t s0 = static_cast<hipStream_t>(stream);
  if (no_alloc && p.mode != CGTP_CHANNELWISE)
    return fail(CGTP_ERR_UNSUPPORTED, "the allocation-free forward runs channelwise plans only");
  if ((st = zero_unreached(p, out, G.n, true, s0, &err, no_alloc)) != CGTP_OK) return fail(st, err);
  if (p.mode == CGTP_FULLY_CONNECTED) {
    if (schedule != CGTP_STREAMED)
      return fail(CGTP_ERR_UNSUPPORTED, "fully connected mode runs the streamed schedule only: the conventional one "
                                        "would materialise E x N_w edge weights");
    st = cgtp::uvw_forward(p, G, d, x, pos, shift, phi, A, out, workspace, s0, &err, state);
    return st == CGTP_OK ? ok() : fail(st, err);
  }
  if (state && schedule != CGTP_CONVENTIONAL)
    return fail(CGTP_ERR_UNSUPPORTED, "channelwise plans keep their edge rows in the conventional forward only");
  const char* fam = state ? "fwdk" : schedule == CGTP_STREAMED ? "fwds" : "fwd";
  hipFunction_t kprep, kfwd;
  if ((st = cgtp::get_kernel(p, fam, "cgtp_prep", &kprep, &err, no_alloc)) != CGTP_OK) return fail(st, err);
  if ((st = cgtp::get_kernel(p, fam, schedule == CGTP_STREAMED ? "cgtp_fwd_streamed" : "cgtp_fwd", &kfwd, &err,
                             no_alloc)) != CGTP_OK)
    return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const cgtp::TaskGroups tg = cgtp::task_groups(cgtp::forward_tasks(p));
  const int ngroup = int(tg.tasks.size());
  // With a state buffer every edge's row goes there, in one receiver chunk.
  void* G_ws = state ? state : workspace;
  const std::vector<std::pair<int, int>> fchunks =
      !state ? G.chunks(g_chunk_edges(p, G, budget))
             : G.n > 0 ? std::vector<std::pair<int, int>>{{0, G.n}} : std::vector<std::pair<int, int>>{};
  for (auto& c : fchunks) {
    int i0 = c.first, nrec = c.second - c.first;
    int e0 = G.row_ptr[c.first], e1 = G.row_ptr[c.second];
    if (e1 > e0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &e0, &e1, &G_ws};
      if ((st = cgtp::launch(kprep, unsigned((e1 - e0 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    int per = (nrec + 7) / 8;
    // Heaviest-first slot order: valid for a launch over every receiver (per = ceil(N / 8)).
    const int32_t* ord = (i0 == 0 && nrec == G.n) ? d.rorder : nullptr;
    void* b[] = {(void*)&x, (void*)&phi, (void*)&A, &G_ws, (void*)&d.row_ptr, (void*)&d.col, &out, &i0, &nrec, &per, &e0,
                 (void*)&ord};
    if ((st = cgtp::launch(kfwd, unsigned(8 * ngroup * per), 64 * cgtp::fwd_split(p) * tg.ncb, 0, s, b, &err)) != CGTP_OK)
      return fail(st, err);
  }
  return ok();
}

cgtp_status_t cgtp_conv_forward(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                void* workspace, size_t ws_bytes, void* stream) {
  return conv_forward_impl(plan, g, schedule, x, pos, shift, phi, A, out, workspace, ws_bytes, stream, nullptr,
                           plan ? plan->p.scratch_budget : 0, false);
}

}  // extern "C"

namespace cgtp {
cgtp_status_t forward_in_scratch(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                 const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                 void* scratch, size_t scratch_bytes, void* stream) {
  return conv_forward_impl(plan, g, schedule, x, pos, shift, phi, A, out, scratch, scratch_bytes, stream, nullptr,
                           scratch_bytes, true);
}
}  // namespace cgtp

extern "C" {

cgtp_status_t cgtp_state_size(cgtp_plan_t plan, cgtp_graph_t g, size_t* bytes) {
  if (!plan || !g || !bytes) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  const cgtp::Plan& p = plan->p;
  if (p.mode == CGTP_FULLY_CONNECTED)
    *bytes = std::max<size_t>(cgtp::uvw_state_bytes(p, g->g), 256);
  else {  // channelwise: the backward's per-edge rows (G, then Y) of every edge
    // A row longer than the N_w edge weights would make the kept state larger than the E x N_w
    // weight tensor the streamed design exists to avoid (high-l plans: 5,196 values per edge
    // against N_w = 3,392 at l <= 6 with 32 channels); such plans recompute the rows instead.
    if (cgtp::bwd_row_stride(p) > p.n_w)
      return fail(CGTP_ERR_UNSUPPORTED, "the per-edge rows (" + std::to_string(cgtp::bwd_row_stride(p)) +
                                            " values) are longer than the N_w = " + std::to_string(p.n_w) +
                                            " edge weights: keeping them is refused, the backward recomputes them");
    *bytes = std::max<size_t>(size_t(g->g.e) * size_t(cgtp::bwd_row_stride(p)) * p.elem(), 256);
  }
  return ok();
}

cgtp_status_t cgtp_conv_forward_keep_state(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                           const void* shift, const void* phi, const void* A, void* out, void* state,
                                           size_t state_bytes, void* workspace, size_t ws_bytes, void* stream) {
  size_t need = 0;
  cgtp_status_t st = cgtp_state_size(plan, g, &need);
  if (st != CGTP_OK) return st;
  if (!state || state_bytes < need) return fail(CGTP_ERR_WORKSPACE, "state buffer too small (cgtp_state_size)");
  const cgtp_schedule_t sched = plan->p.mode == CGTP_FULLY_CONNECTED ? CGTP_STREAMED : CGTP_CONVENTIONAL;
  return conv_forward_impl(plan, g, sched, x, pos, shift, phi, A, out, workspace, ws_bytes, stream, state,
                           plan->p.scratch_budget, false);
}

}  // extern "C"


extern "C" {

static cgtp_status_t conv_backward_impl(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                        const void* shift, const void* phi, const void* A, const void* grad_out,
                                        void* grad_x, void* grad_pos, void* grad_edge_vec, void* grad_phi,
                                        void* grad_A, void* workspace, size_t ws_bytes, void* stream,
                                        const void* state) {
  if (!plan || !g) return fail(CGTP_ERR_INVALID_ARG, "null plan or graph");
  if (!x || !pos || !A || !grad_out) return fail(CGTP_ERR_INVALID_ARG, "null input tensor");
  cgtp::Plan& p = plan->p;
  cgtp::Graph& G = g->g;
  if ((phi == nullptr) != (p.radial != 0))
    return fail(CGTP_ERR_INVALID_ARG, p.radial ? "phi must be NULL: the plan computes the radial basis"
                                               : "null phi (the plan has no radial basis of its own)");
  if (!grad_x && !grad_pos && !grad_edge_vec && !grad_phi && !grad_A) return ok();
  size_t need = 0;
  cgtp_workspace_size(plan, g, CGTP_OP_BACKWARD, &need);
  if (!workspace || ws_bytes < need) return fail(CGTP_ERR_WORKSPACE, "workspace too small");
  std::string err;
  cgtp::DeviceGraph d;
  cgtp_status_t st = cgtp::device_graph(G, &d, &err);
  if (st != CGTP_OK) return fail(st, err);
  if (grad_x && (st = zero_unreached(p, grad_x, G.n, false, static_cast<hipStream_t>(stream), &err)) != CGTP_OK)
    return fail(st, err);
  if (p.mode == CGTP_FULLY_CONNECTED) {
    st = cgtp::uvw_backward(p, G, d, x, pos, shift, phi, A, grad_out, grad_x, grad_pos, grad_edge_vec,
                            grad_phi, grad_A, workspace, static_cast<hipStream_t>(stream), &err, state);
    return st == CGTP_OK ? ok() : fail(st, err);
  }
  BwdLayout L = bwd_layout(p, G);
  hipFunction_t kzero, kprep, krecv, ksrc, kfinal, kpos, kred;
  const char* fam = "bwd";
  if ((st = cgtp::get_kernel(p, fam, "cgtp_fill_zero", &kzero, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_prep", &kprep, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_bwd_recv", &krecv, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_bwd_src", &ksrc, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_edge_final", &kfinal, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_pos_grad", &kpos, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_a_reduce", &kred, &err)) != CGTP_OK)
    return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* Gb = ws + L.g_off;
  void* ep = ws + L.ep_off;
  void* ap = ws + L.ap_off;
  void* gev = grad_edge_vec ? grad_edge_vec : static_cast<void*>(ws + L.gev_off);
  const bool need_edge = grad_edge_vec || grad_pos || grad_phi;
  void* gev_arg = (grad_edge_vec || grad_pos) ? gev : nullptr;
  // With one receiver chunk every A-bar slot is written (not accumulated) by its workgroup.
  int acc_slots = L.chunks.size() > 1 ? 1 : 0;
  if (grad_A && acc_slots) {
    long long n = (long long)L.nslot * p.K * p.n_w;
    void* a[] = {&ap, &n};
    if ((st = cgtp::launch(kzero, unsigned((n + 255) / 256), 256, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  }
  const int nt_r = L.ntask_r;
  const cgtp::TaskGroups tsrc = cgtp::task_groups(cgtp::source_tasks(p));
  int eps = int(L.emax);
  for (size_t c = 0; c < L.chunks.size(); ++c) {
    int i0 = L.chunks[c].first, nrec = L.chunks[c].second - L.chunks[c].first;
    int e0 = G.row_ptr[L.chunks[c].first], e1 = G.row_ptr[L.chunks[c].second];
    if (state) {  // the rows the forward kept, for every edge: this chunk's start
      Gb = const_cast<char*>(static_cast<const char*>(state)) + size_t(e0) * size_t(cgtp::bwd_row_stride(p)) * p.elem();
    } else if (e1 > e0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &e0, &e1, &Gb};
      if ((st = cgtp::launch(kprep, unsigned((e1 - e0 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    if (need_edge || grad_A) {
      int per, nch;
      chunk_geometry(nrec, &per, &nch);
      const int32_t* ord = (i0 == 0 && nrec == G.n) ? d.rorder : nullptr;
      void* a[] = {(void*)&x, (void*)&phi, (void*)&A, &Gb, (void*)&d.row_ptr, (void*)&d.col, (void*)&grad_out,
                   &ep, &ap, &i0, &nrec, &per, &nch, &e0, &eps, &acc_slots, (void*)&ord};
      if ((st = cgtp::launch(krecv, unsigned(8 * nt_r * nch), 64 * kRecvGroup, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    if (grad_x) {
      int n = G.n, per = (G.n + 7) / 8, acc = c > 0 ? 1 : 0;
      void *sb = nullptr, *se = nullptr;
      if ((st = source_bounds(p, fam, G, d, L, c, ws, s, &sb, &se, &err)) != CGTP_OK) return fail(st, err);
      void* a[] = {(void*)&phi, (void*)&A, &Gb, (void*)&grad_out, (void*)&d.recv, &sb, &se, (void*)&d.src_edge,
                   &grad_x, &n, &per, &e0, &acc, (void*)&d.sorder};
      if ((st = cgtp::launch(ksrc, unsigned(8 * tsrc.tasks.size() * per), 64 * kSrcSplit * tsrc.ncb, 0, s, a, &err)) !=
          CGTP_OK)
        return fail(st, err);
    }
    if (need_edge && e1 > e0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &ep, &e0, &e1, &eps, &grad_phi,
                   &gev_arg};
      if ((st = cgtp::launch(kfinal, unsigned((e1 - e0 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
  }
  if (grad_pos) {
    int n = G.n;
    void* a[] = {&gev, (void*)&d.row_ptr, (void*)&d.src_ptr, (void*)&d.src_edge, &n, &grad_pos};
    if ((st = cgtp::launch(kpos, unsigned(n), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  }
  if (grad_A) {
    int n = p.K * p.n_w, ns = L.nslot;
    void* a[] = {&ap, &ns, &n, &grad_A};
    if ((st = cgtp::launch(kred, unsigned((n + 63) / 64), 512, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  }
  return ok();
}

cgtp_status_t cgtp_conv_backward(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos, const void* shift,
                                 const void* phi, const void* A, const void* grad_out, void* grad_x, void* grad_pos,
                                 void* grad_edge_vec, void* grad_phi, void* grad_A, void* workspace, size_t ws_bytes,
                                 void* stream) {
  return conv_backward_impl(plan, g, x, pos, shift, phi, A, grad_out, grad_x, grad_pos, grad_edge_vec, grad_phi,
                            grad_A, workspace, ws_bytes, stream, nullptr);
}

cgtp_status_t cgtp_conv_backward_with_state(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                            const void* shift, const void* phi, const void* A, const void* grad_out,
                                            const void* state, size_t state_bytes, void* grad_x, void* grad_pos,
                                            void* grad_edge_vec, void* grad_phi, void* grad_A, void* workspace,
                                            size_t ws_bytes, void* stream) {
  size_t need = 0;
  cgtp_status_t st = cgtp_state_size(plan, g, &need);
  if (st != CGTP_OK) return st;
  if (!state || state_bytes < need) return fail(CGTP_ERR_WORKSPACE, "state buffer too small (cgtp_state_size)");
  return conv_backward_impl(plan, g, x, pos, shift, phi, A, grad_out, grad_x, grad_pos, grad_edge_vec, grad_phi,
                            grad_A, workspace, ws_bytes, stream, state);
}

cgtp_status_t cgtp_conv_double_backward(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                        const void* shift, const void* phi, const void* A, const void* grad_out,
                                        const void* v_x, const void* v_pos, const void* v_edge_vec,
                                        const void* v_phi, const void* v_A, void* gg_x, void* gg_pos,
                                        void* gg_edge_vec, void* gg_phi, void* gg_A, void* gg_grad_out,
                                        void* workspace, size_t ws_bytes, void* stream) {
  if (!plan || !g) return fail(CGTP_ERR_INVALID_ARG, "null plan or graph");
  if (!x || !pos || !A || !grad_out) return fail(CGTP_ERR_INVALID_ARG, "null input tensor");
  cgtp::Plan& p = plan->p;
  cgtp::Graph& G = g->g;
  if ((phi == nullptr) != (p.radial != 0))
    return fail(CGTP_ERR_INVALID_ARG, p.radial ? "phi must be NULL: the plan computes the radial basis"
                                               : "null phi (the plan has no radial basis of its own)");
  if (p.radial && v_phi)
    return fail(CGTP_ERR_INVALID_ARG, "v_phi must be NULL with an in-kernel radial basis: the radial values' "
                                      "direction follows from v_edge_vec and v_pos");
  if (!gg_x && !gg_pos && !gg_edge_vec && !gg_phi && !gg_A && !gg_grad_out) return ok();
  size_t need = 0;
  cgtp_status_t st = cgtp_workspace_size(plan, g, CGTP_OP_DOUBLE_BACKWARD, &need);
  if (st != CGTP_OK) return st;
  if (!workspace || ws_bytes < need) return fail(CGTP_ERR_WORKSPACE, "workspace too small");
  std::string err;
  cgtp::DeviceGraph d;
  if ((st = cgtp::device_graph(G, &d, &err)) != CGTP_OK) return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.mode == CGTP_FULLY_CONNECTED && p.radial) {
    // phi and phidot = phi'(|r|) (r-hat . rdot) per edge, the double backward on the plain twin
    // with them as inputs (its gg_phi and the first-order phi-bar kept), then the radial terms
    // of e-bar-dot and the position sums.
    cgtp::Plan* pp = nullptr;
    if ((st = plain_plan(p, &pp, &err)) != CGTP_OK) return fail(st, err);
    const RadialDblLayout R = radial_dbl_layout(p, *pp, G);
    char* ws = static_cast<char*>(workspace);
    void* phi_a = ws + R.phi_off;
    void* vphi_a = ws + R.vphi_off;
    void* gphi = gg_phi ? gg_phi : static_cast<void*>(ws + R.gphi_off);
    void* pb = ws + R.pb_off;
    const bool want_ev = gg_edge_vec || gg_pos;
    void* gev = gg_edge_vec ? gg_edge_vec : static_cast<void*>(ws + R.gev_off);
    hipFunction_t kvals, kdedge, kpos;
    if ((st = cgtp::get_kernel(p, "uvw_rdbl", "cgtp_radial_vals", &kvals, &err)) != CGTP_OK ||
        (st = cgtp::get_kernel(p, "uvw_rdbl", "cgtp_radial_dedge", &kdedge, &err)) != CGTP_OK ||
        (st = cgtp::get_kernel(p, "uvw_rdbl", "cgtp_pos_grad", &kpos, &err)) != CGTP_OK)
      return fail(st, err);
    int e0 = 0, e1 = G.e;
    if (e1 > 0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&v_edge_vec, (void*)&v_pos,
                   &e0, &e1, &phi_a, &vphi_a};
      if ((st = cgtp::launch(kvals, unsigned((e1 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
    }
    st = cgtp::uvw_double_backward(*pp, G, d, x, pos, shift, phi_a, A, grad_out, v_x, v_pos, v_edge_vec, vphi_a, v_A,
                                   gg_x, nullptr, want_ev ? gev : nullptr, gphi, gg_A, gg_grad_out,
                                   ws + R.inner_off, s, &err, want_ev ? pb : nullptr);
    if (st != CGTP_OK) return fail(st, err);
    if (want_ev && e1 > 0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&v_edge_vec, (void*)&v_pos,
                   &gphi, &pb, &e0, &e1, &gev};
      if ((st = cgtp::launch(kdedge, unsigned((e1 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
    }
    if (gg_pos) {
      int n = G.n;
      void* a[] = {&gev, (void*)&d.row_ptr, (void*)&d.src_ptr, (void*)&d.src_edge, &n, &gg_pos};
      if ((st = cgtp::launch(kpos, unsigned(n), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
    }
    return ok();
  }
  if (p.mode == CGTP_FULLY_CONNECTED) {
    st = cgtp::uvw_double_backward(p, G, d, x, pos, shift, phi, A, grad_out, v_x, v_pos, v_edge_vec, v_phi, v_A, gg_x,
                                   gg_pos, gg_edge_vec, gg_phi, gg_A, gg_grad_out, workspace, s, &err);
    return st == CGTP_OK ? ok() : fail(st, err);
  }
  if (gg_x && (st = zero_unreached(p, gg_x, G.n, false, s, &err)) != CGTP_OK) return fail(st, err);
  if (gg_grad_out && (st = zero_unreached(p, gg_grad_out, G.n, true, s, &err)) != CGTP_OK) return fail(st, err);
  BwdLayout L = dbl_layout(p, G);
  hipFunction_t kzero, kprep, kfwd, krecv, ksrc, kfinal, kpos, kred;
  const char* fam = "dbl";
  if ((st = cgtp::get_kernel(p, fam, "cgtp_fill_zero", &kzero, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_prep2", &kprep, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_dfwd", &kfwd, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_drecv", &krecv, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_dsrc", &ksrc, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_dedge_final", &kfinal, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_pos_grad", &kpos, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam, "cgtp_a_reduce", &kred, &err)) != CGTP_OK)
    return fail(st, err);
  // A missing direction is read from a primal array of the same shape with a zero scale.
  const bool f64 = p.dtype == CGTP_F64;
  // With an in-kernel radial basis the radial tangent is computed (Gdot rows), never absent.
  double sxd = v_x ? 1.0 : 0.0, sphid = (v_phi || p.radial) ? 1.0 : 0.0, sAd = v_A ? 1.0 : 0.0;
  float sxf = float(sxd), sphif = float(sphid), sAf = float(sAd);
  void* psx = f64 ? (void*)&sxd : (void*)&sxf;
  void* psphi = f64 ? (void*)&sphid : (void*)&sphif;
  void* psA = f64 ? (void*)&sAd : (void*)&sAf;
  const void* vx = v_x ? v_x : x;
  const void* vphi = v_phi ? v_phi : phi;
  const void* vA = v_A ? v_A : A;
  char* ws = static_cast<char*>(workspace);
  void* Gb = ws + L.g_off;
  void* ep = ws + L.ep_off;
  void* ap = ws + L.ap_off;
  void* gev = gg_edge_vec ? gg_edge_vec : static_cast<void*>(ws + L.gev_off);
  const bool need_edge = gg_edge_vec || gg_pos || gg_phi;
  void* gev_arg = (gg_edge_vec || gg_pos) ? gev : nullptr;
  if (gg_A) {
    long long n = (long long)L.nslot * p.K * p.n_w;
    void* a[] = {&ap, &n};
    if ((st = cgtp::launch(kzero, unsigned((n + 255) / 256), 256, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  }
  const int nt_f = int(cgtp::forward_tasks(p).size()), nt_r = L.ntask_r, nt_s = L.ntask_s;
  int eps = int(L.emax);
  for (size_t c = 0; c < L.chunks.size(); ++c) {
    int i0 = L.chunks[c].first, nrec = L.chunks[c].second - L.chunks[c].first;
    int e0 = G.row_ptr[L.chunks[c].first], e1 = G.row_ptr[L.chunks[c].second];
    if (e1 > e0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&v_edge_vec, (void*)&v_pos,
                   &e0, &e1, &Gb};
      if ((st = cgtp::launch(kprep, unsigned((e1 - e0 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    void* out_arg = gg_grad_out;
    void* common[] = {(void*)&x, (void*)&vx, (void*)&phi, (void*)&vphi, (void*)&A, (void*)&vA, &Gb,
                      (void*)&d.row_ptr, (void*)&d.col, (void*)&grad_out, &out_arg, &ep, &ap, psx, psphi, psA};
    const int32_t* ord = (i0 == 0 && nrec == G.n) ? d.rorder : nullptr;
    if (gg_grad_out) {
      int per = (nrec + 7) / 8;
      void* a[21];
      std::copy(common, common + 16, a);
      a[16] = &i0; a[17] = &nrec; a[18] = &per; a[19] = &e0; a[20] = (void*)&ord;
      if ((st = cgtp::launch(kfwd, unsigned(8 * nt_f * per), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
    }
    if (need_edge || gg_A) {
      int per, nch;
      chunk_geometry(nrec, &per, &nch);
      void* a[23];
      std::copy(common, common + 16, a);
      a[16] = &i0; a[17] = &nrec; a[18] = &per; a[19] = &nch; a[20] = &e0; a[21] = &eps; a[22] = (void*)&ord;
      if ((st = cgtp::launch(krecv, unsigned(8 * nt_r * nch), 64 * kRecvGroup, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    if (gg_x) {
      int n = G.n, per = (G.n + 7) / 8, acc = c > 0 ? 1 : 0;
      void *sb = nullptr, *se = nullptr;
      if ((st = source_bounds(p, fam, G, d, L, c, ws, s, &sb, &se, &err)) != CGTP_OK) return fail(st, err);
      void* a[] = {(void*)&phi, (void*)&vphi, (void*)&A, (void*)&vA, &Gb, (void*)&grad_out, (void*)&d.recv, &sb, &se,
                   (void*)&d.src_edge, &gg_x, psphi, psA, &n, &per, &e0, &acc, (void*)&d.sorder};
      if ((st = cgtp::launch(ksrc, unsigned(8 * nt_s * per), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
    }
    if (need_edge && e1 > e0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&v_edge_vec, (void*)&v_pos,
                   &ep, &e0, &e1, &eps, &gg_phi, &gev_arg};
      if ((st = cgtp::launch(kfinal, unsigned((e1 - e0 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
  }
  if (gg_pos) {
    int n = G.n;
    void* a[] = {&gev, (void*)&d.row_ptr, (void*)&d.src_ptr, (void*)&d.src_edge, &n, &gg_pos};
    if ((st = cgtp::launch(kpos, unsigned(n), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  }
  if (gg_A) {
    int n = p.K * p.n_w, ns = L.nslot;
    void* a[] = {&ap, &ns, &n, &gg_A};
    if ((st = cgtp::launch(kred, unsigned((n + 63) / 64), 512, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  }
  return ok();
}

// Third-order derivative (LunaTP Appendix F, Algorithm 4): the gradients of
// S3 = <q, second-order outputs> as the sum over the ten 4-linear terms below, each evaluated by
// the backward's passes on the 2K plan with one slot open: the source pass for the node slot a,
// the forward for the cotangent slot d, the receiver pass for the edge-operand slot b and, through
// phi-bar = A_k H and A-bar = phi_k^T H, for the weight factors.
namespace {
enum TriVar { TV_X, TV_Y, TV_PHI, TV_A, TV_G, TV_VX, TV_VY, TV_VPHI, TV_VA, TV_QX, TV_QY, TV_QPHI, TV_QA, TV_QG, TV_N };
struct TriTerm {
  int a, b, f[2][2], d;
};
// (a, b, weight factors (phi-type, A-type) x2, d); -1 = no second factor.
const TriTerm kTriTerms[10] = {
    {TV_VX, TV_QY, {{TV_PHI, TV_A}, {-1, -1}}, TV_G},
    {TV_VX, TV_Y, {{TV_QPHI, TV_A}, {TV_PHI, TV_QA}}, TV_G},
    {TV_VX, TV_Y, {{TV_PHI, TV_A}, {-1, -1}}, TV_QG},
    {TV_QX, TV_VY, {{TV_PHI, TV_A}, {-1, -1}}, TV_G},
    {TV_X, TV_VY, {{TV_QPHI, TV_A}, {TV_PHI, TV_QA}}, TV_G},
    {TV_X, TV_VY, {{TV_PHI, TV_A}, {-1, -1}}, TV_QG},
    {TV_QX, TV_Y, {{TV_VPHI, TV_A}, {TV_PHI, TV_VA}}, TV_G},
    {TV_X, TV_QY, {{TV_VPHI, TV_A}, {TV_PHI, TV_VA}}, TV_G},
    {TV_X, TV_Y, {{TV_VPHI, TV_QA}, {TV_QPHI, TV_VA}}, TV_G},
    {TV_X, TV_Y, {{TV_VPHI, TV_A}, {TV_PHI, TV_VA}}, TV_QG},
};
}  // namespace

cgtp_status_t cgtp_conv_triple_backward(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* Y,
                                        const void* phi, const void* A, const void* grad_out, const void* v_x,
                                        const void* v_Y, const void* v_phi, const void* v_A, const void* q_x,
                                        const void* q_Y, const void* q_phi, const void* q_A, const void* q_grad_out,
                                        void* t_x, void* t_Y, void* t_phi, void* t_A, void* t_grad_out, void* t_vx,
                                        void* t_vY, void* t_vphi, void* t_vA, void* workspace, size_t ws_bytes,
                                        void* stream) {
  if (!plan || !g) return fail(CGTP_ERR_INVALID_ARG, "null plan or graph");
  if (!x || !Y || !phi || !A || !grad_out) return fail(CGTP_ERR_INVALID_ARG, "null input tensor");
  cgtp::Plan& p = plan->p;
  cgtp::Graph& G = g->g;
  if (p.mode != CGTP_CHANNELWISE) return fail(CGTP_ERR_UNSUPPORTED, "the triple backward is channelwise only");
  if (p.radial) return fail(CGTP_ERR_UNSUPPORTED, "the triple backward takes phi as an input (no fused radial basis)");
  const void* in[TV_N] = {x, Y, phi, A, grad_out, v_x, v_Y, v_phi, v_A, q_x, q_Y, q_phi, q_A, q_grad_out};
  void* out[TV_N] = {t_x, t_Y, t_phi, t_A, t_grad_out, t_vx, t_vY, t_vphi, t_vA,
                     nullptr, nullptr, nullptr, nullptr, nullptr};
  bool any = false;
  for (int k = 0; k < TV_QX; ++k) any = any || out[k];
  if (!any) return ok();
  std::string err;
  cgtp::Plan* tpp = nullptr;
  cgtp_status_t st = tri_plan(p, &tpp, &err);
  if (st != CGTP_OK) return fail(st, err);
  cgtp::Plan& tp = *tpp;
  const TriLayout T = tri_layout(p, tp, G);
  if (!workspace || ws_bytes < T.total) return fail(CGTP_ERR_WORKSPACE, "workspace too small");
  cgtp::DeviceGraph d;
  if ((st = cgtp::device_graph(G, &d, &err)) != CGTP_OK) return fail(st, err);
  const char* fam = "tri";
  hipFunction_t kzero, kprep, kfwd, krecv, ksrc, kfinal, kred, kpphi, kpa;
  if ((st = cgtp::get_kernel(tp, fam, "cgtp_fill_zero", &kzero, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_prep_y", &kprep, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_fwd", &kfwd, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_bwd_recv", &krecv, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_bwd_src", &ksrc, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_edge_final_y", &kfinal, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_tri_a_reduce", &kred, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_tri_pack_phi", &kpphi, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(tp, fam, "cgtp_tri_pack_a", &kpa, &err)) != CGTP_OK)
    return fail(st, err);
  // The same passes with the plan's own K, for terms with one weight factor (no stacking).
  hipFunction_t k1fwd, k1recv, k1src, k1final, k1red;
  const char* fam1 = "tri1";
  if ((st = cgtp::get_kernel(p, fam1, "cgtp_fwd", &k1fwd, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam1, "cgtp_bwd_recv", &k1recv, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam1, "cgtp_bwd_src", &k1src, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam1, "cgtp_edge_final_y", &k1final, &err)) != CGTP_OK ||
      (st = cgtp::get_kernel(p, fam1, "cgtp_tri_a_reduce", &k1red, &err)) != CGTP_OK)
    return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int K = p.K, K2 = tp.K, SH = p.sh_dim, NW = p.n_w, el = int(p.elem());
  char* ws = static_cast<char*>(workspace);
  auto zero = [&](void* buf, long long n) -> cgtp_status_t {
    if (!buf || n <= 0) return CGTP_OK;
    void* a[] = {&buf, &n};
    return cgtp::launch(kzero, unsigned((n + 255) / 256), 256, 0, s, a, &err);
  };
  // Outputs are sums over terms: zeroed first, then every pass adds into them.
  const long long sizes[TV_QX] = {(long long)G.n * p.c_in, (long long)G.e * SH, (long long)G.e * K,
                                  (long long)K * NW, (long long)G.n * p.c_out, (long long)G.n * p.c_in,
                                  (long long)G.e * SH, (long long)G.e * K, (long long)K * NW};
  for (int k = 0; k < TV_QX; ++k)
    if ((st = zero(out[k], sizes[k])) != CGTP_OK) return fail(st, err);
  void* apk = ws + T.ak_off;
  void* ep = ws + T.L.ep_off;
  void* ap = ws + T.L.ap_off;
  void* pk = ws + T.pk_off;
  void* Gb = ws + T.gy_off[0];
  const BwdLayout& L = T.L;
  int eps = int(L.emax);
  auto rows_at = [&](void* base, int e0, int width) -> void* {
    return base ? static_cast<char*>(base) + (size_t)e0 * width * el : nullptr;
  };
  for (size_t c = 0; c < L.chunks.size(); ++c) {
    int i0 = L.chunks[c].first, nrec = L.chunks[c].second - L.chunks[c].first;
    int e0 = G.row_ptr[L.chunks[c].first], e1 = G.row_ptr[L.chunks[c].second];
    void *sb = nullptr, *se = nullptr;
    bool bounds_done = false;
    const int32_t* ord = (i0 == 0 && nrec == G.n) ? d.rorder : nullptr;
    // Terms grouped by their edge operand: one operand's rows are in the workspace at a time.
    for (int bvar : {TV_Y, TV_VY, TV_QY}) {
      if (!in[bvar]) continue;
      bool rows_ready = false;
      for (const TriTerm& tt : kTriTerms) {
        if (tt.b != bvar) continue;
        const void* fp[2] = {nullptr, nullptr};
        const void* fa[2] = {nullptr, nullptr};
        bool live = false;
        for (int k = 0; k < 2; ++k)
          if (tt.f[k][0] >= 0 && in[tt.f[k][0]] && in[tt.f[k][1]]) {
            fp[k] = in[tt.f[k][0]];
            fa[k] = in[tt.f[k][1]];
            live = true;
          }
        if (!live || !in[tt.a] || !in[tt.d]) continue;
        void* dphi[2] = {nullptr, nullptr};
        void* dA[2] = {nullptr, nullptr};
        for (int k = 0; k < 2; ++k)
          if (fp[k]) {
            dphi[k] = out[tt.f[k][0]];
            dA[k] = out[tt.f[k][1]];
          }
        const bool want_a = out[tt.a] != nullptr, want_d = out[tt.d] != nullptr, want_b = out[tt.b] != nullptr;
        const bool want_pb = dphi[0] || dphi[1], want_ab = dA[0] || dA[1];
        if (!want_a && !want_d && !want_b && !want_pb && !want_ab) continue;
        if (!rows_ready && e1 > e0) {
          const void* yop = in[bvar];
          void* a[] = {(void*)&yop, &e0, &e1, &Gb};
          if ((st = cgtp::launch(kprep, unsigned((e1 - e0 + 63) / 64), 64, 0, s, a, &err)) != CGTP_OK)
            return fail(st, err);
        }
        rows_ready = true;
        // One live weight factor: the plan's own kernels take it as (phi, A).  Two: the 2K plan's
        // kernels take the stacked factors [phi_1 | phi_2] (chunk rows) and [A_1; A_2].
        const int one = fp[0] && fp[1] ? -1 : fp[0] ? 0 : 1;
        const cgtp::Plan& kp = one >= 0 ? p : tp;
        hipFunction_t kf = one >= 0 ? k1fwd : kfwd, kr = one >= 0 ? k1recv : krecv;
        hipFunction_t ks = one >= 0 ? k1src : ksrc, kfi = one >= 0 ? k1final : kfinal;
        hipFunction_t krd = one >= 0 ? k1red : kred;
        const void* phi_arg = nullptr;
        const void* a_arg = nullptr;
        if (one >= 0) {
          phi_arg = fp[one];
          a_arg = fa[one];
          if (one == 1) {   // the stacked kernels' first half carries it in the single-factor ones
            dphi[0] = dphi[1];
            dA[0] = dA[1];
          }
          dphi[1] = dA[1] = nullptr;
        } else {
          if (e1 > e0) {
            void* a[] = {(void*)&fp[0], (void*)&fp[1], &e0, &e1, &pk};
            long long n = (long long)(e1 - e0) * K2;
            if ((st = cgtp::launch(kpphi, unsigned((n + 255) / 256), 256, 0, s, a, &err)) != CGTP_OK)
              return fail(st, err);
          }
          void* a[] = {(void*)&fa[0], (void*)&fa[1], &apk};
          long long n = (long long)K2 * NW;
          if ((st = cgtp::launch(kpa, unsigned((n + 255) / 256), 256, 0, s, a, &err)) != CGTP_OK)
            return fail(st, err);
          // The kernels index the radial values by sorted edge: shift the chunk's packed rows to e0.
          phi_arg = static_cast<const char*>(pk) - (ptrdiff_t)e0 * K2 * el;
          a_arg = apk;
        }
        const void* av = in[tt.a];
        const void* dv = in[tt.d];
        if (want_a) {   // node slot open: the source pass, added into the output
          if (!bounds_done) {
            if ((st = source_bounds(tp, fam, G, d, L, c, ws, s, &sb, &se, &err)) != CGTP_OK) return fail(st, err);
            bounds_done = true;
          }
          const cgtp::TaskGroups tsrc = cgtp::task_groups(cgtp::source_tasks(kp));
          int n = G.n, per = (G.n + 7) / 8, acc = 1;
          void* dst = out[tt.a];
          void* a[] = {(void*)&phi_arg, (void*)&a_arg, &Gb, (void*)&dv, (void*)&d.recv, &sb, &se, (void*)&d.src_edge,
                       &dst, &n, &per, &e0, &acc, (void*)&d.sorder};
          if ((st = cgtp::launch(ks, unsigned(8 * tsrc.tasks.size() * per), 64 * kSrcSplit * tsrc.ncb, 0, s, a,
                                 &err)) != CGTP_OK)
            return fail(st, err);
        }
        if (want_d && nrec > 0) {   // cotangent slot open: the forward, added into the output rows
          const cgtp::TaskGroups tg = cgtp::task_groups(cgtp::forward_tasks(kp));
          int per = (nrec + 7) / 8;
          void* dst = out[tt.d];
          void* a[] = {(void*)&av, (void*)&phi_arg, (void*)&a_arg, &Gb, (void*)&d.row_ptr, (void*)&d.col, &dst, &i0,
                       &nrec, &per, &e0, (void*)&ord};
          if ((st = cgtp::launch(kf, unsigned(8 * tg.tasks.size() * per), 64 * cgtp::fwd_split(kp) * tg.ncb, 0, s,
                                 a, &err)) != CGTP_OK)
            return fail(st, err);
        }
        if ((want_b || want_pb || want_ab) && nrec > 0) {   // edge-operand and weight slots: the receiver pass
          int per, nch, acc_slots = 0;
          chunk_geometry(nrec, &per, &nch);
          const int ntask_r = int(cgtp::recv_backward_tasks(kp).size());
          void* a[] = {(void*)&av, (void*)&phi_arg, (void*)&a_arg, &Gb, (void*)&d.row_ptr, (void*)&d.col, (void*)&dv,
                       &ep, &ap, &i0, &nrec, &per, &nch, &e0, &eps, &acc_slots, (void*)&ord};
          if ((st = cgtp::launch(kr, unsigned(8 * ntask_r * nch), 64 * kRecvGroup, 0, s, a, &err)) != CGTP_OK)
            return fail(st, err);
          if (e1 > e0 && (want_b || want_pb)) {   // d/dphi_k = A_k H: half k of phi-bar; Y-bar of slot b
            void* g1 = rows_at(dphi[0], e0, K);
            void* g2 = rows_at(dphi[1], e0, K);
            void* gy = want_b ? rows_at(out[tt.b], e0, SH) : nullptr;
            void* b[] = {&ep, &e0, &e1, &g1, &g2, &gy};
            if ((st = cgtp::launch(kfi, unsigned((e1 - e0 + 63) / 64), 64, 0, s, b, &err)) != CGTP_OK)
              return fail(st, err);
          }
          if (want_ab) {   // d/dA_k = phi_k^T H: rows k K .. k K + K - 1 of this pass's A-bar
            int ns = 8 * nch;   // the slots this chunk's receiver pass wrote
            void* b[] = {&ap, &ns, &dA[0], &dA[1]};
            if ((st = cgtp::launch(krd, unsigned((kp.K * NW + 63) / 64), 512, 0, s, b, &err)) != CGTP_OK)
              return fail(st, err);
          }
        }
      }
    }
  }
  return ok();
}

cgtp_status_t cgtp_check_edges(cgtp_plan_t plan, cgtp_graph_t g, const void* pos, const void* shift, void* workspace,
                               size_t ws_bytes, void* stream, int* first_bad) {
  if (!plan || !g || !pos || !first_bad) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  cgtp::Plan& p = plan->p;
  cgtp::Graph& G = g->g;
  *first_bad = -1;
  if (G.e == 0) return ok();
  const int nblk = (G.e + 255) / 256;
  if (!workspace || ws_bytes < size_t(nblk) * sizeof(int))
    return fail(CGTP_ERR_WORKSPACE, "workspace smaller than 4 bytes per 256 edges");
  std::string err;
  cgtp::DeviceGraph d;
  cgtp_status_t st = cgtp::device_graph(G, &d, &err);
  if (st != CGTP_OK) return fail(st, err);
  hipFunction_t k;
  const char* fam = p.mode == CGTP_CHANNELWISE ? "fwd" : "uvw_fwd";
  if ((st = cgtp::get_kernel(p, fam, "cgtp_check_edges", &k, &err)) != CGTP_OK) return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int ne = G.e;
  void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &ne, &workspace};
  if ((st = cgtp::launch(k, unsigned(nblk), 256, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
  std::vector<int> h(size_t(nblk), 0);
  if (hipMemcpyAsync(h.data(), workspace, h.size() * sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(CGTP_ERR_HIP, "copying the edge check result failed");
  int m = 0x7fffffff;
  for (int v : h) m = std::min(m, v);
  if (m == 0x7fffffff) return ok();
  *first_bad = m;
  return fail(CGTP_ERR_DEGENERATE_EDGE, "edge " + std::to_string(m) + " (receiver-sorted) has zero length");
}

cgtp_status_t cgtp_layout_convert(cgtp_plan_t plan, int side, int direction, int n_nodes, const void* src, void* dst,
                                  void* stream) {
  if (!plan) return fail(CGTP_ERR_INVALID_ARG, "null plan");
  if (side != 0 && side != 1) return fail(CGTP_ERR_INVALID_ARG, "side must be 0 (input) or 1 (output)");
  if (direction != 0 && direction != 1) return fail(CGTP_ERR_INVALID_ARG, "direction must be 0 or 1");
  if (n_nodes < 0) return fail(CGTP_ERR_INVALID_ARG, "negative node count");
  if (n_nodes == 0) return ok();
  if (!src || !dst) return fail(CGTP_ERR_INVALID_ARG, "null tensor argument");
  if (src == dst) return fail(CGTP_ERR_INVALID_ARG, "src and dst must not overlap");
  cgtp::Plan& p = plan->p;
  std::string err;
  hipFunction_t k;
  cgtp_status_t st = cgtp::get_kernel(p, "layout", side == 0 ? "cgtp_layout_in" : "cgtp_layout_out", &k, &err);
  if (st != CGTP_OK) return fail(st, err);
  long long total = (long long)n_nodes * (side == 0 ? p.c_in : p.c_out);
  int to_mul_ir = direction;
  void* a[] = {(void*)&src, &dst, &total, &to_mul_ir};
  st = cgtp::launch(k, unsigned((total + 255) / 256), 256, 0, static_cast<hipStream_t>(stream), a, &err);
  return st == CGTP_OK ? ok() : fail(st, err);
}

}  // extern "C"

extern "C" {

cgtp_status_t cgtp_profile_begin(void) {
  cgtp::profile_begin();
  return ok();
}

cgtp_status_t cgtp_profile_end(void) {
  std::string err;
  cgtp_status_t st = cgtp::profile_end(&err);
  return st == CGTP_OK ? ok() : fail(st, err);
}

int cgtp_profile_count(void) { return int(cgtp::profile_entries().size()); }

cgtp_status_t cgtp_profile_get(int index, char* name, int capacity, long long* launches, double* total_ms) {
  auto v = cgtp::profile_entries();
  if (index < 0 || index >= int(v.size())) return fail(CGTP_ERR_INVALID_ARG, "profile index out of range");
  if (name && capacity > 0) {
    std::snprintf(name, size_t(capacity), "%s", v[index].name.c_str());
  }
  if (launches) *launches = v[index].launches;
  if (total_ms) *total_ms = v[index].ms;
  return ok();
}

}  // extern "C"
