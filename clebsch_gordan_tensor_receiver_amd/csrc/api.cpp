// The extern "C" surface declared in include/cgtp.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "cgtp.h"
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

// Edges of G rows that fit in the scratch budget (at least the largest in-degree).
long long g_chunk_edges(const cgtp::Plan& p, const cgtp::Graph& g) {
  long long row = (long long)p.g_stride * (long long)p.elem();
  long long cap = std::max<long long>(1, (long long)(p.scratch_budget / size_t(row)));
  return std::max<long long>(cap, g.max_in_degree);
}

long long max_chunk_edges(const cgtp::Graph& g, const std::vector<std::pair<int, int>>& ch) {
  long long m = 0;
  for (auto& c : ch) m = std::max<long long>(m, g.row_ptr[c.second] - g.row_ptr[c.first]);
  return m;
}

// Launch geometry shared with the generated kernels (codegen.cpp).
constexpr int kSrcSplit = 2;    // waves per sender in the source backward
constexpr int kRecvGroup = 4;   // receivers (one wave each) per workgroup in the receiver backward

// Workspace plan of a backward call.
struct BwdLayout {
  long long cap = 0;            // edges per receiver chunk
  std::vector<std::pair<int, int>> chunks;
  int ntask_r = 0, ntask_s = 0, V = 0, row = 0;
  int nslot = 0;                // A-bar partial slots (max over chunks)
  long long emax = 0;           // edges of the largest chunk (stride of the edge partials)
  size_t g_off = 0, ep_off = 0, ap_off = 0, gev_off = 0, total = 0;
};

// Receivers per XCD and receiver groups per XCD of a chunk; the groups are the A-bar slots.
void chunk_geometry(int nrec, int* per, int* nch) {
  *per = (nrec + 7) / 8;
  *nch = (*per + kRecvGroup - 1) / kRecvGroup;
}

BwdLayout bwd_layout(const cgtp::Plan& p, const cgtp::Graph& g) {
  BwdLayout L;
  L.ntask_r = int(cgtp::recv_backward_tasks(p).size());
  L.ntask_s = int(cgtp::source_tasks(p).size());
  L.V = 0;
  L.row = cgtp::recv_partial_row(p);
  const int grow = cgtp::bwd_row_stride(p);
  long long row_bytes = (long long)(grow + L.row) * (long long)p.elem();
  L.cap = std::max<long long>(std::max<long long>(1, (long long)(p.scratch_budget / size_t(row_bytes))),
                              g.max_in_degree);
  L.chunks = g.chunks(L.cap);
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
  off += align256(size_t(L.nslot) * size_t(p.K) * size_t(p.n_w) * p.elem());
  L.gev_off = off;
  off += align256(size_t(std::max(g.e, 1)) * 3 * p.elem());
  L.total = off;
  return L;
}

// Workspace plan of a double-backward call: G and Gdot rows (2 g_stride per edge), the edge
// partials of the receiver pass, A-bar-dot slots and an edge-vector buffer.
BwdLayout dbl_layout(const cgtp::Plan& p, const cgtp::Graph& g) {
  BwdLayout L;
  L.ntask_r = int(cgtp::dbl_recv_tasks(p).size());
  L.ntask_s = int(cgtp::source_tasks(p).size());
  L.V = 0;
  L.row = cgtp::dbl_partial_row(p);
  long long row_bytes = (long long)(2 * p.g_stride + L.row) * (long long)p.elem();
  L.cap = std::max<long long>(std::max<long long>(1, (long long)(p.scratch_budget / size_t(row_bytes))),
                              g.max_in_degree);
  L.chunks = g.chunks(L.cap);
  long long emax = std::max<long long>(1, max_chunk_edges(g, L.chunks));
  L.emax = emax;
  for (auto& c : L.chunks) {
    int per, nch;
    chunk_geometry(c.second - c.first, &per, &nch);
    L.nslot = std::max(L.nslot, 8 * nch);
  }
  size_t off = 0;
  L.g_off = off;
  off += align256(size_t(emax) * size_t(2 * p.g_stride) * p.elem());
  L.ep_off = off;
  off += align256(size_t((emax + 63) / 64 * 64) * size_t(L.row) * p.elem());  // tiles of 64 edges
  L.ap_off = off;
  off += align256(size_t(L.nslot) * size_t(p.K) * size_t(p.n_w) * p.elem());
  L.gev_off = off;
  off += align256(size_t(std::max(g.e, 1)) * 3 * p.elem());
  L.total = off;
  return L;
}

// Feature blocks that no path reaches (output side) or leaves (input side) are not written by
// the kernels; zero the whole tensor first when such a block exists.
cgtp_status_t zero_unreached(cgtp::Plan& p, void* buf, int n, bool out_side, hipStream_t s, std::string* err) {
  const auto& blocks = out_side ? p.out : p.in;
  const auto& by = out_side ? p.by_out : p.by_in;
  bool any = false;
  for (size_t k = 0; k < blocks.size(); ++k) any = any || by[k].empty();
  if (!any) return CGTP_OK;
  const char* fam = p.mode == CGTP_CHANNELWISE ? "fwd" : "uvw_fwd";
  hipFunction_t kz;
  cgtp_status_t st = cgtp::get_kernel(p, fam, "cgtp_fill_zero", &kz, err);
  if (st != CGTP_OK) return st;
  long long cnt = (long long)n * (out_side ? p.c_out : p.c_in);
  void* a[] = {&buf, &cnt};
  return cgtp::launch(kz, unsigned((cnt + 255) / 256), 256, 0, s, a, err);
}

}  // namespace

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
  } else {
    if (ops & (1 << CGTP_OP_DOUBLE_BACKWARD))
      return fail(CGTP_ERR_UNSUPPORTED, "double backward is channelwise only");
    if (ops & (1 << CGTP_OP_FORWARD)) fams.push_back("uvw_fwd");
    if (ops & (1 << CGTP_OP_BACKWARD)) fams.push_back("uvw_bwd");
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
  for (auto& kv : g->g.views) {
    (void)hipSetDevice(kv.first.first);
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
    if (op == CGTP_OP_DOUBLE_BACKWARD) return fail(CGTP_ERR_UNSUPPORTED, "double backward is channelwise only");
    *bytes = std::max<size_t>(cgtp::uvw_workspace(p, G, op), 256);
    return ok();
  }
  if (op == CGTP_OP_FORWARD) {
    auto ch = G.chunks(g_chunk_edges(p, G));
    need = align256(size_t(max_chunk_edges(G, ch)) * size_t(p.g_stride) * p.elem());
  } else if (op == CGTP_OP_BACKWARD) {
    need = bwd_layout(p, G).total;
  } else {
    need = dbl_layout(p, G).total;
  }
  *bytes = std::max<size_t>(need, 256);
  return ok();
}

static cgtp_status_t conv_forward_impl(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                       const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                       void* workspace, size_t ws_bytes, void* stream, void* state) {
  if (!plan || !g) return fail(CGTP_ERR_INVALID_ARG, "null plan or graph");
  if (!x || !pos || !A || !out) return fail(CGTP_ERR_INVALID_ARG, "null tensor argument");
  if (schedule != CGTP_STREAMED && schedule != CGTP_CONVENTIONAL) return fail(CGTP_ERR_INVALID_ARG, "bad schedule");
  cgtp::Plan& p = plan->p;
  if ((phi == nullptr) != (p.radial != 0))
    return fail(CGTP_ERR_INVALID_ARG, p.radial ? "phi must be NULL: the plan computes the radial basis"
                                               : "null phi (the plan has no radial basis of its own)");
  cgtp::Graph& G = g->g;
  size_t need = 0;
  cgtp_workspace_size(plan, g, CGTP_OP_FORWARD, &need);
  if (ws_bytes < need || (!workspace && need > 0)) return fail(CGTP_ERR_WORKSPACE, "workspace too small");
  std::string err;
  cgtp::DeviceGraph d;
  cgtp_status_t st = cgtp::device_graph(G, &d, &err);
  if (st != CGTP_OK) return fail(st, err);
  hipStream_t s0 = static_cast<hipStream_t>(stream);
  if ((st = zero_unreached(p, out, G.n, true, s0, &err)) != CGTP_OK) return fail(st, err);
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
  if ((st = cgtp::get_kernel(p, fam, "cgtp_prep", &kprep, &err)) != CGTP_OK) return fail(st, err);
  if ((st = cgtp::get_kernel(p, fam, schedule == CGTP_STREAMED ? "cgtp_fwd_streamed" : "cgtp_fwd", &kfwd, &err)) !=
      CGTP_OK)
    return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const cgtp::TaskGroups tg = cgtp::task_groups(cgtp::forward_tasks(p));
  const int ngroup = int(tg.tasks.size());
  // With a state buffer every edge's row goes there, in one receiver chunk.
  void* G_ws = state ? state : workspace;
  const std::vector<std::pair<int, int>> fchunks =
      !state ? G.chunks(g_chunk_edges(p, G))
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
    void* b[] = {(void*)&x, (void*)&phi, (void*)&A, &G_ws, (void*)&d.row_ptr, (void*)&d.col, &out, &i0, &nrec, &per, &e0};
    if ((st = cgtp::launch(kfwd, unsigned(8 * ngroup * per), 64 * cgtp::fwd_split(p) * tg.ncb, 0, s, b, &err)) != CGTP_OK)
      return fail(st, err);
  }
  return ok();
}

cgtp_status_t cgtp_conv_forward(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                void* workspace, size_t ws_bytes, void* stream) {
  return conv_forward_impl(plan, g, schedule, x, pos, shift, phi, A, out, workspace, ws_bytes, stream, nullptr);
}

cgtp_status_t cgtp_state_size(cgtp_plan_t plan, cgtp_graph_t g, size_t* bytes) {
  if (!plan || !g || !bytes) return fail(CGTP_ERR_INVALID_ARG, "null argument");
  const cgtp::Plan& p = plan->p;
  if (p.mode == CGTP_FULLY_CONNECTED)
    *bytes = std::max<size_t>(cgtp::uvw_state_bytes(p, g->g), 256);
  else  // channelwise: the backward's per-edge rows (G, then Y) of every edge
    *bytes = std::max<size_t>(size_t(g->g.e) * size_t(cgtp::bwd_row_stride(p)) * p.elem(), 256);
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
  return conv_forward_impl(plan, g, sched, x, pos, shift, phi, A, out, workspace, ws_bytes, stream, state);
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
    st = cgtp::uvw_backward(p, G, d, nullptr, x, pos, shift, phi, A, grad_out, grad_x, grad_pos, grad_edge_vec,
                            grad_phi, grad_A, workspace, static_cast<hipStream_t>(stream), &err, state);
    return st == CGTP_OK ? ok() : fail(st, err);
  }
  BwdLayout L = bwd_layout(p, G);
  const cgtp::SourceViews* views = nullptr;
  if (grad_x && (st = cgtp::source_views(G, L.cap, &views, &err)) != CGTP_OK) return fail(st, err);
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
      void* a[] = {(void*)&x, (void*)&phi, (void*)&A, &Gb, (void*)&d.row_ptr, (void*)&d.col, (void*)&grad_out,
                   &ep, &ap, &i0, &nrec, &per, &nch, &e0, &eps, &acc_slots};
      if ((st = cgtp::launch(krecv, unsigned(8 * nt_r * nch), 64 * kRecvGroup, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    if (grad_x) {
      int n = G.n, per = (G.n + 7) / 8, acc = c > 0 ? 1 : 0;
      void* sp = static_cast<int32_t*>(views->base) + views->ptr_off[c];
      void* se = static_cast<int32_t*>(views->base) + views->edge_off[c];
      void* a[] = {(void*)&phi, (void*)&A, &Gb, (void*)&grad_out, (void*)&d.recv, &sp, &se, &grad_x, &n, &per, &e0,
                   &acc};
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
  if (!x || !pos || !phi || !A || !grad_out) return fail(CGTP_ERR_INVALID_ARG, "null input tensor");
  cgtp::Plan& p = plan->p;
  cgtp::Graph& G = g->g;
  if (p.mode != CGTP_CHANNELWISE) return fail(CGTP_ERR_UNSUPPORTED, "double backward is channelwise only");
  if (p.radial) return fail(CGTP_ERR_UNSUPPORTED, "double backward takes phi as an input (no fused radial basis)");
  if (!gg_x && !gg_pos && !gg_edge_vec && !gg_phi && !gg_A && !gg_grad_out) return ok();
  size_t need = 0;
  cgtp_status_t st = cgtp_workspace_size(plan, g, CGTP_OP_DOUBLE_BACKWARD, &need);
  if (st != CGTP_OK) return st;
  if (!workspace || ws_bytes < need) return fail(CGTP_ERR_WORKSPACE, "workspace too small");
  std::string err;
  cgtp::DeviceGraph d;
  if ((st = cgtp::device_graph(G, &d, &err)) != CGTP_OK) return fail(st, err);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (gg_x && (st = zero_unreached(p, gg_x, G.n, false, s, &err)) != CGTP_OK) return fail(st, err);
  if (gg_grad_out && (st = zero_unreached(p, gg_grad_out, G.n, true, s, &err)) != CGTP_OK) return fail(st, err);
  BwdLayout L = dbl_layout(p, G);
  const cgtp::SourceViews* views = nullptr;
  if (gg_x && (st = cgtp::source_views(G, L.cap, &views, &err)) != CGTP_OK) return fail(st, err);
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
  double sxd = v_x ? 1.0 : 0.0, sphid = v_phi ? 1.0 : 0.0, sAd = v_A ? 1.0 : 0.0;
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
    if (gg_grad_out) {
      int per = (nrec + 7) / 8;
      void* a[20];
      std::copy(common, common + 16, a);
      a[16] = &i0; a[17] = &nrec; a[18] = &per; a[19] = &e0;
      if ((st = cgtp::launch(kfwd, unsigned(8 * nt_f * per), 64, 0, s, a, &err)) != CGTP_OK) return fail(st, err);
    }
    if (need_edge || gg_A) {
      int per, nch;
      chunk_geometry(nrec, &per, &nch);
      void* a[22];
      std::copy(common, common + 16, a);
      a[16] = &i0; a[17] = &nrec; a[18] = &per; a[19] = &nch; a[20] = &e0; a[21] = &eps;
      if ((st = cgtp::launch(krecv, unsigned(8 * nt_r * nch), 64 * kRecvGroup, 0, s, a, &err)) != CGTP_OK)
        return fail(st, err);
    }
    if (gg_x) {
      int n = G.n, per = (G.n + 7) / 8, acc = c > 0 ? 1 : 0;
      void* sp = static_cast<int32_t*>(views->base) + views->ptr_off[c];
      void* se = static_cast<int32_t*>(views->base) + views->edge_off[c];
      void* a[] = {(void*)&phi, (void*)&vphi, (void*)&A, (void*)&vA, &Gb, (void*)&grad_out, (void*)&d.recv, &sp, &se,
                   &gg_x, psphi, psA, &n, &per, &e0, &acc};
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
