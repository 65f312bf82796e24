// Launch sequences of the fully connected (uvw) streamed convolution.
//
// Workspace per receiver chunk: G rows of the chunk's edges, the receiver states S (and for the
// backward Sbar, the per-edge partial sums and the A-bar row-slice partials); per sender chunk:
// G rows of the chunk's out-edges in source order and the source states Z.  Chunks are sized so
// that this stays within the plan's scratch budget: the workspace never scales with E x N_w.
#include "uvw_launch.hpp"

#include <algorithm>

#include "kernels.hpp"

namespace cgtp {
namespace {

size_t al(size_t n) { return (n + 255) / 256 * 256; }

// Greedy ranges [a, b) of nodes whose cost (per node + per edge of the node's list) fits `budget`.
std::vector<std::pair<int, int>> ranges(int n, const std::vector<int32_t>& ptr, size_t per_node, size_t per_edge,
                                        size_t budget) {
  std::vector<std::pair<int, int>> out;
  int a = 0;
  while (a < n) {
    int b = a + 1;
    while (b < n) {
      size_t cost = size_t(b + 1 - a) * per_node + size_t(ptr[b + 1] - ptr[a]) * per_edge;
      if (cost > budget) break;
      ++b;
    }
    out.push_back({a, b});
    a = b;
  }
  return out;
}

constexpr int kAbarSplit = 32;  // row slices of the A-bar GEMM per group (fixed-order partial sums)
constexpr int kMaxSplit = 8;    // K slices of the forward and x-bar GEMMs (64 output columns: few row tiles)

// K slices of a GEMM with M rows, N columns and depth Kd: enough workgroups to fill the chip
// (about 1,024), slices of at least 128, at most kMaxSplit.  Returns the slice length in *kper.
int gemm_split(int M, int N, int Kd, int* kper) {
  const long long tiles = (long long)((M + 63) / 64) * ((N + 63) / 64);
  int ns = int(std::min<long long>(kMaxSplit, std::max<long long>(1, (1024 + tiles - 1) / std::max(1LL, tiles))));
  ns = std::max(1, std::min(ns, Kd / 128));
  int kp = (Kd + ns - 1) / ns;
  kp = (kp + 31) / 32 * 32;
  *kper = kp;
  return (Kd + kp - 1) / kp;
}

// Largest d x mul over the sides: rows per node times columns of a split-K partial.
size_t max_side_cols(const std::vector<UvwSideInfo>& sides) {
  size_t m = 1;
  for (auto& s : sides) m = std::max(m, size_t(s.d) * size_t(s.mul));
  return m;
}

// Waves per receiver for the state and edge kernels of a chunk: doubled (up to kMaxStripes) while
// the chunk's (receiver, task) waves would not give every SIMD four; for the state kernel the
// partial states of the extra waves must fit 64 KiB of LDS.
int stripes(int nrec, int ntask, size_t lds_per_extra_wave) {
  const long long waves = 8LL * ((nrec + 7) / 8) * ntask;
  int n = 1;
  while (n < kMaxStripes && waves * n < 4096 && size_t(2 * n - 1) * lds_per_extra_wave <= (64u << 10)) n *= 2;
  return n;
}

struct UvwPlanB {
  UvwLayout L;
  std::vector<std::pair<int, int>> rchunks, schunks;
  int V = 0, ep_row = 0;
  long long emax = 1, kmax = 1;
  int nmax = 1, jmax = 1;
  size_t g_off = 0, s_off = 0, sb_off = 0, ep_off = 0, ap_off = 0, z_off = 0, xp_off = 0, gs_off = 0, gev_off = 0;
  size_t total = 0;
};

UvwPlanB layout_bwd(const Plan& p, const Graph& g) {
  UvwPlanB B;
  B.L = uvw_layout(p);
  const size_t el = p.elem();
  B.V = edge_partial_width(p);
  B.ep_row = B.L.n_state_tasks * B.V;
  const size_t per_recv = 2 * size_t(B.L.recv_stride) * el;
  const size_t per_edge = (size_t(p.g_stride) + size_t(B.ep_row)) * el;
  B.rchunks = ranges(g.n, g.row_ptr, per_recv, per_edge, p.scratch_budget);
  for (auto& c : B.rchunks) {
    B.emax = std::max<long long>(B.emax, g.row_ptr[c.second] - g.row_ptr[c.first]);
    B.nmax = std::max(B.nmax, c.second - c.first);
  }
  B.schunks = ranges(g.n, g.src_ptr, (size_t(B.L.send_stride) + kMaxSplit * max_side_cols(B.L.send)) * el,
                     size_t(p.g_stride) * el, p.scratch_budget);
  for (auto& c : B.schunks) {
    B.kmax = std::max<long long>(B.kmax, g.src_ptr[c.second] - g.src_ptr[c.first]);
    B.jmax = std::max(B.jmax, c.second - c.first);
  }
  size_t dmax = 1;
  for (auto& s : B.L.recv) dmax = std::max(dmax, size_t(s.D) * size_t(s.mul));
  // Receiver phase.
  size_t off = 0;
  B.g_off = off;
  off += al(size_t(B.emax) * p.g_stride * el);
  B.s_off = off;
  off += al(size_t(B.nmax) * B.L.recv_stride * el);
  B.sb_off = off;
  off += al(size_t(B.nmax) * B.L.recv_stride * el);
  B.ep_off = off;
  off += al(size_t(B.emax) * B.ep_row * el);
  B.ap_off = off;
  off += al(size_t(kAbarSplit) * dmax * el);
  size_t recv_phase = off;
  // Sender phase (reuses the same bytes).
  off = 0;
  B.gs_off = off;
  off += al(size_t(B.kmax) * p.g_stride * el);
  B.z_off = off;
  off += al(size_t(B.jmax) * B.L.send_stride * el);
  B.xp_off = off;
  off += al(size_t(B.jmax) * kMaxSplit * max_side_cols(B.L.send) * el);
  size_t send_phase = off;
  B.gev_off = std::max(recv_phase, send_phase);
  B.total = B.gev_off + al(size_t(std::max(g.e, 1)) * 3 * el);
  return B;
}

struct UvwPlanF {
  UvwLayout L;
  std::vector<std::pair<int, int>> chunks;
  long long emax = 1;
  int nmax = 1;
  size_t g_off = 0, s_off = 0, part_off = 0, total = 0;
};

UvwPlanF layout_fwd(const Plan& p, const Graph& g) {
  UvwPlanF F;
  F.L = uvw_layout(p);
  const size_t el = p.elem();
  F.chunks = ranges(g.n, g.row_ptr, (size_t(F.L.recv_stride) + kMaxSplit * max_side_cols(F.L.recv)) * el,
                    size_t(p.g_stride) * el, p.scratch_budget);
  for (auto& c : F.chunks) {
    F.emax = std::max<long long>(F.emax, g.row_ptr[c.second] - g.row_ptr[c.first]);
    F.nmax = std::max(F.nmax, c.second - c.first);
  }
  F.g_off = 0;
  F.s_off = al(size_t(F.emax) * p.g_stride * el);
  F.part_off = F.s_off + al(size_t(F.nmax) * F.L.recv_stride * el);
  F.total = F.part_off + al(size_t(F.nmax) * kMaxSplit * max_side_cols(F.L.recv) * el);
  return F;
}

// Double backward layout.  Receiver phase per chunk: G and Gdot rows, one state buffer (the terms
// of Sdot one after another, then S), Sbar and Sbar-dot, the forward GEMMs' split-K partials of
// up to four terms per output block (summed by one reduce), four edge-partial buffers and the
// A-bar slices.  Sender phase: source-order G and Gdot rows, Z and the x-bar partials of up to
// three terms.  Beside both: e-bar-dot (when only gg_pos is asked for) and a zero phi-dot.
constexpr int kDblFwdTerms = 4, kDblSrcTerms = 3, kDblEdgeBufs = 4;

struct UvwPlanD {
  UvwLayout L;
  std::vector<std::pair<int, int>> rchunks, schunks;
  int V = 0, ep_row = 0;
  long long emax = 1, kmax = 1;
  int nmax = 1, jmax = 1;
  size_t g_off = 0, gd_off = 0, s_off = 0, sb_off = 0, sbd_off = 0, part_off = 0, ep_off = 0, ap_off = 0;
  size_t gs_off = 0, gsd_off = 0, z_off = 0, xp_off = 0, gev_off = 0, zphi_off = 0, total = 0;
  size_t ep_bytes = 0;
};

size_t sum_side_cols(const std::vector<UvwSideInfo>& sides) {
  size_t m = 0;
  for (auto& s : sides) m += size_t(s.d) * size_t(s.mul);
  return std::max<size_t>(m, 1);
}

UvwPlanD layout_dbl(const Plan& p, const Graph& g) {
  UvwPlanD B;
  B.L = uvw_layout(p);
  const size_t el = p.elem();
  B.V = edge_partial_width(p);
  B.ep_row = B.L.n_state_tasks * B.V;
  const size_t rcols = sum_side_cols(B.L.recv), scols = sum_side_cols(B.L.send);
  const size_t per_recv = (3 * size_t(B.L.recv_stride) + kDblFwdTerms * kMaxSplit * rcols) * el;
  const size_t per_edge = (2 * size_t(p.g_stride) + kDblEdgeBufs * size_t(B.ep_row)) * el;
  B.rchunks = ranges(g.n, g.row_ptr, per_recv, per_edge, p.scratch_budget);
  for (auto& c : B.rchunks) {
    B.emax = std::max<long long>(B.emax, g.row_ptr[c.second] - g.row_ptr[c.first]);
    B.nmax = std::max(B.nmax, c.second - c.first);
  }
  B.schunks = ranges(g.n, g.src_ptr, (size_t(B.L.send_stride) + kDblSrcTerms * kMaxSplit * scols) * el,
                     2 * size_t(p.g_stride) * el, p.scratch_budget);
  for (auto& c : B.schunks) {
    B.kmax = std::max<long long>(B.kmax, g.src_ptr[c.second] - g.src_ptr[c.first]);
    B.jmax = std::max(B.jmax, c.second - c.first);
  }
  size_t dmax = 1;
  for (auto& s : B.L.recv) dmax = std::max(dmax, size_t(s.D) * size_t(s.mul));
  size_t off = 0;
  auto take = [&](size_t* at, size_t bytes) {
    *at = off;
    off += al(bytes);
  };
  take(&B.g_off, size_t(B.emax) * p.g_stride * el);
  take(&B.gd_off, size_t(B.emax) * p.g_stride * el);
  take(&B.s_off, size_t(B.nmax) * B.L.recv_stride * el);
  take(&B.sb_off, size_t(B.nmax) * B.L.recv_stride * el);
  take(&B.sbd_off, size_t(B.nmax) * B.L.recv_stride * el);
  take(&B.part_off, size_t(B.nmax) * kDblFwdTerms * kMaxSplit * rcols * el);
  B.ep_bytes = al(size_t(B.emax) * B.ep_row * el);
  take(&B.ep_off, kDblEdgeBufs * B.ep_bytes);
  take(&B.ap_off, size_t(kAbarSplit) * dmax * el);
  const size_t recv_phase = off;
  off = 0;
  take(&B.gs_off, size_t(B.kmax) * p.g_stride * el);
  take(&B.gsd_off, size_t(B.kmax) * p.g_stride * el);
  take(&B.z_off, size_t(B.jmax) * B.L.send_stride * el);
  take(&B.xp_off, size_t(B.jmax) * kDblSrcTerms * kMaxSplit * scols * el);
  off = std::max(off, recv_phase);
  take(&B.gev_off, size_t(std::max(g.e, 1)) * 3 * el);
  take(&B.zphi_off, size_t(std::max(g.e, 1)) * p.K * el);
  B.total = off;
  return B;
}

unsigned cdiv(long long a, long long b) { return unsigned((a + b - 1) / b); }

cgtp_status_t launch3(hipFunction_t f, unsigned gx, unsigned gy, unsigned gz, unsigned block, hipStream_t s,
                      void** args, std::string* err) {
  return launch_grid(f, gx, gy, gz, block, 0, s, args, err);
}

}  // namespace

size_t uvw_workspace(const Plan& p, const Graph& g, cgtp_op_t op) {
  if (op == CGTP_OP_DOUBLE_BACKWARD) return layout_dbl(p, g).total;
  return op == CGTP_OP_FORWARD ? layout_fwd(p, g).total : layout_bwd(p, g).total;
}

size_t uvw_state_bytes(const Plan& p, const Graph& g) {
  return size_t(g.n) * size_t(uvw_layout(p).recv_stride) * p.elem();
}

cgtp_status_t uvw_forward(Plan& p, Graph& G, const DeviceGraph& d, const void* x, const void* pos, const void* shift,
                          const void* phi, const void* A, void* out, void* workspace, hipStream_t s,
                          std::string* err, void* state) {
  UvwPlanF F = layout_fwd(p, G);
  cgtp_status_t st;
  hipFunction_t kprep, kstate;
  if ((st = get_kernel(p, "uvw_fwd", "cgtp_prep", &kprep, err)) != CGTP_OK ||
      (st = get_kernel(p, "uvw_fwd", "cgtp_uvw_state", &kstate, err)) != CGTP_OK)
    return st;
  std::vector<hipFunction_t> kg, kr;
  for (auto& side : F.L.recv) {
    hipFunction_t f, r;
    const std::string nm = "cgtp_gemm_fwd" + std::to_string(side.blk);
    if ((st = get_kernel(p, "uvw_fwd", nm, &f, err)) != CGTP_OK ||
        (st = get_kernel(p, "uvw_fwd", nm + "_reduce", &r, err)) != CGTP_OK)
      return st;
    kg.push_back(f);
    kr.push_back(r);
  }
  void* Gb = static_cast<char*>(workspace) + F.g_off;
  void* S = static_cast<char*>(workspace) + F.s_off;
  void* part = static_cast<char*>(workspace) + F.part_off;
  for (auto& c : F.chunks) {
    int i0 = c.first, nrec = c.second - c.first;
    int e0 = G.row_ptr[c.first], e1 = G.row_ptr[c.second];
    if (e1 > e0) {
      void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &e0, &e1, &Gb};
      if ((st = launch(kprep, cdiv(e1 - e0, 64), 64, 0, s, a, err)) != CGTP_OK) return st;
    }
    int per = (nrec + 7) / 8;
    const size_t lds_w = size_t(F.L.state_acc) * 64 * p.elem();
    const int nst = stripes(nrec, F.L.n_state_tasks, lds_w);
    void* Sc = state ? static_cast<void*>(static_cast<char*>(state) + size_t(i0) * F.L.recv_stride * p.elem()) : S;
    void* b[] = {(void*)&x, (void*)&phi, &Gb, (void*)&d.row_ptr, (void*)&d.col, &Sc, &i0, &nrec, &per, &e0};
    if ((st = launch(kstate, unsigned(8 * F.L.n_state_tasks * per), 64 * nst, unsigned((nst - 1) * lds_w), s, b,
                     err)) != CGTP_OK)
      return st;
    for (size_t gi = 0; gi < F.L.recv.size(); ++gi) {
      const auto& side = F.L.recv[gi];
      int M = nrec * side.d, Kd = side.D, kper = 0;
      int ns = gemm_split(M, side.mul, Kd, &kper);
      void* a[] = {&Sc, (void*)&A, &part, &i0, &M, &Kd, &kper};
      if ((st = launch3(kg[gi], cdiv(M, 64), cdiv(side.mul, 64), unsigned(ns), 256, s, a, err)) != CGTP_OK)
        return st;
      void* b[] = {&part, &ns, &M, &out, &i0};
      if ((st = launch(kr[gi], cdiv((long long)M * side.mul, 256), 256, 0, s, b, err)) != CGTP_OK) return st;
    }
  }
  // Output blocks without paths stay untouched by the GEMMs: callers get zeros there.
  return CGTP_OK;
}

cgtp_status_t uvw_backward(Plan& p, Graph& G, const DeviceGraph& d, const void* x,
                           const void* pos, const void* shift, const void* phi, const void* A, const void* gout,
                           void* grad_x, void* grad_pos, void* grad_edge_vec, void* grad_phi, void* grad_A,
                           void* workspace, hipStream_t s, std::string* err, const void* state) {
  UvwPlanB B = layout_bwd(p, G);
  cgtp_status_t st;
  const char* fam = "uvw_bwd";
  hipFunction_t kzero, kprep, kstate, kedge, kedge_s, kfinal, kpos, kprep_src, kz;
  if ((st = get_kernel(p, fam, "cgtp_fill_zero", &kzero, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_prep", &kprep, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_state", &kstate, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_edge", &kedge, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_edge_striped", &kedge_s, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_edge_final", &kfinal, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_pos_grad", &kpos, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_prep_src", &kprep_src, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_zstate", &kz, err)) != CGTP_OK)
    return st;
  std::vector<hipFunction_t> ksb, kab, kacc, kxb;
  for (auto& side : B.L.recv) {
    hipFunction_t f1, f2, f3;
    std::string b = std::to_string(side.blk);
    if ((st = get_kernel(p, fam, "cgtp_gemm_sbar" + b, &f1, err)) != CGTP_OK ||
        (st = get_kernel(p, fam, "cgtp_gemm_abar" + b, &f2, err)) != CGTP_OK ||
        (st = get_kernel(p, fam, "cgtp_abar_accum" + b, &f3, err)) != CGTP_OK)
      return st;
    ksb.push_back(f1);
    kab.push_back(f2);
    kacc.push_back(f3);
  }
  std::vector<hipFunction_t> kxr;
  for (auto& side : B.L.send) {
    hipFunction_t f, r;
    const std::string nm = "cgtp_gemm_xbar" + std::to_string(side.blk);
    if ((st = get_kernel(p, fam, nm, &f, err)) != CGTP_OK || (st = get_kernel(p, fam, nm + "_reduce", &r, err)) != CGTP_OK)
      return st;
    kxb.push_back(f);
    kxr.push_back(r);
  }
  char* ws = static_cast<char*>(workspace);
  void* Gb = ws + B.g_off;
  void* S = ws + B.s_off;
  void* Sb = ws + B.sb_off;
  void* ep = ws + B.ep_off;
  void* ap = ws + B.ap_off;
  void* gev = grad_edge_vec ? grad_edge_vec : static_cast<void*>(ws + B.gev_off);
  void* gev_arg = (grad_edge_vec || grad_pos) ? gev : nullptr;
  const bool need_edge = grad_edge_vec || grad_pos || grad_phi;
  int eps = int(B.emax);
  if (grad_A) {
    long long n = (long long)p.K * p.n_w;
    void* a[] = {&grad_A, &n};
    if ((st = launch(kzero, cdiv(n, 256), 256, 0, s, a, err)) != CGTP_OK) return st;
  }
  if (need_edge || grad_A) {
    for (auto& c : B.rchunks) {
      int i0 = c.first, nrec = c.second - c.first;
      int e0 = G.row_ptr[c.first], e1 = G.row_ptr[c.second];
      int per = (nrec + 7) / 8;
      if (e1 > e0) {
        void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &e0, &e1, &Gb};
        if ((st = launch(kprep, cdiv(e1 - e0, 64), 64, 0, s, a, err)) != CGTP_OK) return st;
      }
      // S of the chunk: kept by the forward, or recomputed into the workspace.
      void* Sc = state ? const_cast<char*>(static_cast<const char*>(state)) + size_t(i0) * B.L.recv_stride * p.elem()
                       : S;
      if (grad_A && !state) {
        const size_t lds_w = size_t(B.L.state_acc) * 64 * p.elem();
        const int nst = stripes(nrec, B.L.n_state_tasks, lds_w);
        void* b[] = {(void*)&x, (void*)&phi, &Gb, (void*)&d.row_ptr, (void*)&d.col, &S, &i0, &nrec, &per, &e0};
        if ((st = launch(kstate, unsigned(8 * B.L.n_state_tasks * per), 64 * nst, unsigned((nst - 1) * lds_w), s, b,
                         err)) != CGTP_OK)
          return st;
      }
      for (size_t gi = 0; gi < B.L.recv.size(); ++gi) {
        const auto& side = B.L.recv[gi];
        int M = nrec * side.d, Kd = side.mul, kper = 0;
        void* a[] = {(void*)&gout, (void*)&A, &Sb, &i0, &M, &Kd, &kper};
        const int cols = sbar_panel(side.mul) ? 64 * kSbarPanelTiles : 64;
        if ((st = launch3(ksb[gi], cdiv(M, 64), cdiv(side.D, cols), 1, 256, s, a, err)) != CGTP_OK) return st;
        if (grad_A) {
          int Ma = side.D, Ka = nrec * side.d;
          int kp = std::max(32, (Ka + kAbarSplit - 1) / kAbarSplit);
          kp = (kp + 31) / 32 * 32;
          int nsplit = (Ka + kp - 1) / kp;
          void* b[] = {&Sc, (void*)&gout, &ap, &i0, &Ma, &Ka, &kp};
          if ((st = launch3(kab[gi], cdiv(Ma, 64), cdiv(side.mul, 64), unsigned(nsplit), 256, s, b, err)) != CGTP_OK)
            return st;
          void* c2[] = {&ap, &nsplit, &grad_A};
          if ((st = launch(kacc[gi], cdiv((long long)side.D * side.mul, 256), 256, 0, s, c2, err)) != CGTP_OK)
            return st;
        }
      }
      if (need_edge && e1 > e0) {
        int nst = stripes(nrec, B.L.n_state_tasks, 0);
        void* a[] = {(void*)&x, (void*)&phi, &Gb, (void*)&d.row_ptr, (void*)&d.col, &Sb, &ep, &i0, &nrec, &per, &e0,
                     &eps, &nst};
        if ((st = launch(nst == 1 ? kedge : kedge_s, unsigned(8 * B.L.n_state_tasks * per * nst), 64, 0, s, a, err)) !=
            CGTP_OK)
          return st;
        void* b[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &ep, &e0, &e1, &eps, &grad_phi,
                     &gev_arg};
        if ((st = launch(kfinal, cdiv(e1 - e0, 256), 256, 0, s, b, err)) != CGTP_OK) return st;
      }
    }
  }
  if (grad_x) {
    void* Gs = ws + B.gs_off;
    void* Z = ws + B.z_off;
    for (auto& c : B.schunks) {
      int j0 = c.first, njs = c.second - c.first;
      int k0 = G.src_ptr[c.first], k1 = G.src_ptr[c.second];
      if (k1 > k0) {
        void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&d.src_edge, &k0, &k1, &Gs};
        if ((st = launch(kprep_src, cdiv(k1 - k0, 64), 64, 0, s, a, err)) != CGTP_OK) return st;
      }
      int per = (njs + 7) / 8;
      void* b[] = {(void*)&phi, &Gs, (void*)&gout, (void*)&d.recv, (void*)&d.src_ptr, (void*)&d.src_edge, &Z, &j0,
                   &njs, &per, &k0};
      if ((st = launch(kz, unsigned(8 * B.L.n_z_tasks * per), 64, 0, s, b, err)) != CGTP_OK) return st;
      void* xp = ws + B.xp_off;
      for (size_t bi = 0; bi < B.L.send.size(); ++bi) {
        const auto& side = B.L.send[bi];
        int M = njs * side.d, Kd = side.D, kper = 0;
        int ns = gemm_split(M, side.mul, Kd, &kper);
        void* a[] = {&Z, (void*)&A, &xp, &j0, &M, &Kd, &kper};
        if ((st = launch3(kxb[bi], cdiv(M, 64), cdiv(side.mul, 64), unsigned(ns), 256, s, a, err)) != CGTP_OK)
          return st;
        void* b[] = {&xp, &ns, &M, &grad_x, &j0};
        if ((st = launch(kxr[bi], cdiv((long long)M * side.mul, 256), 256, 0, s, b, err)) != CGTP_OK) return st;
      }
    }
  }
  if (grad_pos) {
    int n = G.n;
    void* a[] = {&gev, (void*)&d.row_ptr, (void*)&d.src_ptr, (void*)&d.src_edge, &n, &grad_pos};
    if ((st = launch(kpos, unsigned(n), 64, 0, s, a, err)) != CGTP_OK) return st;
  }
  return CGTP_OK;
}

cgtp_status_t uvw_double_backward(Plan& p, Graph& G, const DeviceGraph& d, const void* x, const void* pos,
                                  const void* shift, const void* phi, const void* A, const void* gout,
                                  const void* v_x, const void* v_pos, const void* v_edge_vec, const void* v_phi,
                                  const void* v_A, void* gg_x, void* gg_pos, void* gg_edge_vec, void* gg_phi,
                                  void* gg_A, void* gg_grad_out, void* workspace, hipStream_t s, std::string* err,
                                  void* phibar_out) {
  UvwPlanD B = layout_dbl(p, G);
  cgtp_status_t st;
  const char* fam = "uvw_dbl";
  hipFunction_t kzero, kprep, kprepd, kstate, kedge, kedge_s, kfinal, kpos, kprep_src, kprep_srcd, kz;
  if ((st = get_kernel(p, fam, "cgtp_fill_zero", &kzero, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_prep", &kprep, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_prep_dot", &kprepd, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_state", &kstate, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_edge", &kedge, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_edge_striped", &kedge_s, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_dedge_final", &kfinal, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_pos_grad", &kpos, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_prep_src", &kprep_src, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_prep_src_dot", &kprep_srcd, err)) != CGTP_OK ||
      (st = get_kernel(p, fam, "cgtp_uvw_zstate", &kz, err)) != CGTP_OK)
    return st;
  std::vector<hipFunction_t> kfw, kfr, ksb, kab, kacc, kxb, kxr;
  for (auto& side : B.L.recv) {
    hipFunction_t f0, f1, f2, f3, f4;
    const std::string b = std::to_string(side.blk);
    if ((st = get_kernel(p, fam, "cgtp_gemm_fwd" + b, &f0, err)) != CGTP_OK ||
        (st = get_kernel(p, fam, "cgtp_gemm_fwd" + b + "_reduce", &f1, err)) != CGTP_OK ||
        (st = get_kernel(p, fam, "cgtp_gemm_sbar" + b, &f2, err)) != CGTP_OK ||
        (st = get_kernel(p, fam, "cgtp_gemm_abar" + b, &f3, err)) != CGTP_OK ||
        (st = get_kernel(p, fam, "cgtp_abar_accum" + b, &f4, err)) != CGTP_OK)
      return st;
    kfw.push_back(f0);
    kfr.push_back(f1);
    ksb.push_back(f2);
    kab.push_back(f3);
    kacc.push_back(f4);
  }
  for (auto& side : B.L.send) {
    hipFunction_t f, r;
    const std::string nm = "cgtp_gemm_xbar" + std::to_string(side.blk);
    if ((st = get_kernel(p, fam, nm, &f, err)) != CGTP_OK || (st = get_kernel(p, fam, nm + "_reduce", &r, err)) != CGTP_OK)
      return st;
    kxb.push_back(f);
    kxr.push_back(r);
  }
  const size_t el = p.elem();
  char* ws = static_cast<char*>(workspace);
  void* Gb = ws + B.g_off;
  void* Gdb = ws + B.gd_off;
  void* S = ws + B.s_off;
  void* Sb = ws + B.sb_off;
  void* Sbd = ws + B.sbd_off;
  char* part = ws + B.part_off;
  void* ap = ws + B.ap_off;
  void* gev = gg_edge_vec ? gg_edge_vec : static_cast<void*>(ws + B.gev_off);
  void* gev_arg = (gg_edge_vec || gg_pos) ? gev : nullptr;
  // phibar_out (nullable): the first-order phi-bar per edge (E x K), from the first-order pass.
  const bool need_edge = gg_edge_vec || gg_pos || gg_phi || phibar_out;
  const bool rdir = v_pos || v_edge_vec;
  auto zero = [&](void* ptr, long long n) {
    void* a[] = {&ptr, &n};
    return launch(kzero, cdiv(n, 256), 256, 0, s, a, err);
  };
  // Outputs that some blocks or chunks leave untouched, and the zero phi-dot of a missing v_phi.
  if (gg_A && (st = zero(gg_A, (long long)p.K * p.n_w)) != CGTP_OK) return st;
  if (gg_grad_out && (st = zero(gg_grad_out, (long long)G.n * p.c_out)) != CGTP_OK) return st;
  if (gg_x && (st = zero(gg_x, (long long)G.n * p.c_in)) != CGTP_OK) return st;
  const void* vphi = v_phi;
  if (!vphi && need_edge) {
    void* zp = ws + B.zphi_off;
    if ((st = zero(zp, (long long)std::max(G.e, 1) * p.K)) != CGTP_OK) return st;
    vphi = zp;
  }
  int eps = int(B.emax);
  // Receiver-side terms of Sdot = sum_e phidot T + phi Tdot (Tdot from xdot and from Gdot): their
  // states feed m-dot (times A) and A-bar-dot (S^T mbar); the last term, S times Adot, feeds m-dot.
  struct Term {
    const void *x, *phi;
    void* G;
    const void* A;
    bool abar;
  };
  if (gg_grad_out || gg_A || need_edge) {
    for (auto& c : B.rchunks) {
      int i0 = c.first, nrec = c.second - c.first;
      int e0 = G.row_ptr[c.first], e1 = G.row_ptr[c.second];
      int per = (nrec + 7) / 8;
      if (e1 > e0) {
        void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, &e0, &e1, &Gb};
        if ((st = launch(kprep, cdiv(e1 - e0, 64), 64, 0, s, a, err)) != CGTP_OK) return st;
        void* b[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&v_edge_vec, (void*)&v_pos,
                     &e0, &e1, &Gdb};
        if ((st = launch(kprepd, cdiv(e1 - e0, 64), 64, 0, s, b, err)) != CGTP_OK) return st;
      }
      if (gg_grad_out || gg_A) {
        std::vector<Term> terms;
        if (v_phi) terms.push_back({x, v_phi, Gb, A, true});
        if (v_x) terms.push_back({v_x, phi, Gb, A, true});
        if (rdir) terms.push_back({x, phi, Gdb, A, true});
        if (v_A && gg_grad_out) terms.push_back({x, phi, Gb, v_A, false});
        std::vector<size_t> pbase;  // per output block: first byte of its terms' partials
        std::vector<int> nsplit, kpers;
        size_t acc = 0;
        for (auto& side : B.L.recv) {
          int M = nrec * side.d, kper = 0;
          int ns = gemm_split(M, side.mul, side.D, &kper);
          pbase.push_back(acc);
          nsplit.push_back(ns);
          kpers.push_back(kper);
          acc += size_t(kDblFwdTerms) * ns * size_t(M) * side.mul * el;
        }
        const size_t lds_w = size_t(B.L.state_acc) * 64 * el;
        const int nst = stripes(nrec, B.L.n_state_tasks, lds_w);
        for (size_t t = 0; t < terms.size(); ++t) {
          const Term& T = terms[t];
          void* b[] = {(void*)&T.x, (void*)&T.phi, (void*)&T.G, (void*)&d.row_ptr, (void*)&d.col, &S, &i0, &nrec,
                       &per, &e0};
          if ((st = launch(kstate, unsigned(8 * B.L.n_state_tasks * per), 64 * nst, unsigned((nst - 1) * lds_w), s,
                           b, err)) != CGTP_OK)
            return st;
          for (size_t gi = 0; gi < B.L.recv.size(); ++gi) {
            const auto& side = B.L.recv[gi];
            int M = nrec * side.d, Kd = side.D, kper = kpers[gi], ns = nsplit[gi];
            if (gg_grad_out) {
              void* pt = part + pbase[gi] + t * size_t(ns) * size_t(M) * side.mul * el;
              void* a[] = {&S, (void*)&T.A, &pt, &i0, &M, &Kd, &kper};
              if ((st = launch3(kfw[gi], cdiv(M, 64), cdiv(side.mul, 64), unsigned(ns), 256, s, a, err)) != CGTP_OK)
                return st;
            }
            if (gg_A && T.abar) {
              int Ma = side.D, Ka = nrec * side.d;
              int kp = std::max(32, (Ka + kAbarSplit - 1) / kAbarSplit);
              kp = (kp + 31) / 32 * 32;
              int nsa = (Ka + kp - 1) / kp;
              void* a[] = {&S, (void*)&gout, &ap, &i0, &Ma, &Ka, &kp};
              if ((st = launch3(kab[gi], cdiv(Ma, 64), cdiv(side.mul, 64), unsigned(nsa), 256, s, a, err)) != CGTP_OK)
                return st;
              void* c2[] = {&ap, &nsa, &gg_A};
              if ((st = launch(kacc[gi], cdiv((long long)side.D * side.mul, 256), 256, 0, s, c2, err)) != CGTP_OK)
                return st;
            }
          }
        }
        const int nt = gg_grad_out ? int(terms.size()) : 0;
        if (nt > 0) {
          for (size_t gi = 0; gi < B.L.recv.size(); ++gi) {
            const auto& side = B.L.recv[gi];
            int M = nrec * side.d, ns = nsplit[gi] * nt;
            void* pt = part + pbase[gi];
            void* b[] = {&pt, &ns, &M, &gg_grad_out, &i0};
            if ((st = launch(kfr[gi], cdiv((long long)M * side.mul, 256), 256, 0, s, b, err)) != CGTP_OK) return st;
          }
        }
      }
      if (need_edge && e1 > e0) {
        // Sbar = mbar A^T and Sbar-dot = mbar Adot^T, then the edge passes:
        //   a: (Sbar-dot, phi, x, G), b: (Sbar, phi, xdot, G), c: (Sbar, phidot, x, Gdot) -- their
        //   phi-bar columns sum to phi-bar-dot, their Y-bar columns to Y-bar-dot;
        //   w: (Sbar, phi, x, G) -- the first-order Y-bar of the curvature term.
        for (size_t gi = 0; gi < B.L.recv.size(); ++gi) {
          const auto& side = B.L.recv[gi];
          int M = nrec * side.d, Kd = side.mul, kper = 0;
          const int cols = sbar_panel(side.mul) ? 64 * kSbarPanelTiles : 64;
          void* a[] = {(void*)&gout, (void*)&A, &Sb, &i0, &M, &Kd, &kper};
          if ((st = launch3(ksb[gi], cdiv(M, 64), cdiv(side.D, cols), 1, 256, s, a, err)) != CGTP_OK) return st;
          if (v_A) {
            void* b[] = {(void*)&gout, (void*)&v_A, &Sbd, &i0, &M, &Kd, &kper};
            if ((st = launch3(ksb[gi], cdiv(M, 64), cdiv(side.D, cols), 1, 256, s, b, err)) != CGTP_OK) return st;
          }
        }
        char* ep0 = ws + B.ep_off;
        void* epa = v_A ? ep0 : nullptr;
        void* epb = v_x ? ep0 + B.ep_bytes : nullptr;
        void* epc = ep0 + 2 * B.ep_bytes;
        void* epw = (gev_arg || phibar_out) ? ep0 + 3 * B.ep_bytes : nullptr;
        int nst = stripes(nrec, B.L.n_state_tasks, 0);
        auto edge = [&](const void* xx, const void* ff, void* gg, void* sb, void* ep) {
          void* a[] = {(void*)&xx, (void*)&ff, &gg, (void*)&d.row_ptr, (void*)&d.col, &sb, &ep, &i0, &nrec, &per,
                       &e0, &eps, &nst};
          return launch(nst == 1 ? kedge : kedge_s, unsigned(8 * B.L.n_state_tasks * per * nst), 64, 0, s, a, err);
        };
        if (epa && (st = edge(x, phi, Gb, Sbd, epa)) != CGTP_OK) return st;
        if (epb && (st = edge(v_x, phi, Gb, Sb, epb)) != CGTP_OK) return st;
        if ((st = edge(x, vphi, Gdb, Sb, epc)) != CGTP_OK) return st;
        if (epw && (st = edge(x, phi, Gb, Sb, epw)) != CGTP_OK) return st;
        void* b[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&v_edge_vec, (void*)&v_pos,
                     &epa, &epb, &epc, &epw, &e0, &e1, &eps, &gg_phi, &gev_arg, &phibar_out};
        if ((st = launch(kfinal, cdiv(e1 - e0, 64), 64, 0, s, b, err)) != CGTP_OK) return st;
      }
    }
  }
  // x-bar-dot = Zdot A + Z Adot with Zdot = sum phidot G mbar + phi Gdot mbar (source order).
  if (gg_x && (v_phi || rdir || v_A)) {
    void* Gs = ws + B.gs_off;
    void* Gsd = ws + B.gsd_off;
    void* Z = ws + B.z_off;
    char* xp = ws + B.xp_off;
    for (auto& c : B.schunks) {
      int j0 = c.first, njs = c.second - c.first;
      int k0 = G.src_ptr[c.first], k1 = G.src_ptr[c.second];
      if (k1 > k0) {
        void* a[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&d.src_edge, &k0, &k1, &Gs};
        if ((st = launch(kprep_src, cdiv(k1 - k0, 64), 64, 0, s, a, err)) != CGTP_OK) return st;
        void* b[] = {(void*)&pos, (void*)&shift, (void*)&d.recv, (void*)&d.col, (void*)&d.src_edge,
                     (void*)&v_edge_vec, (void*)&v_pos, &k0, &k1, &Gsd};
        if ((st = launch(kprep_srcd, cdiv(k1 - k0, 64), 64, 0, s, b, err)) != CGTP_OK) return st;
      }
      struct ZTerm {
        const void* phi;
        void* G;
        const void* A;
      };
      std::vector<ZTerm> terms;
      if (v_phi) terms.push_back({v_phi, Gs, A});
      if (rdir) terms.push_back({phi, Gsd, A});
      if (v_A) terms.push_back({phi, Gs, v_A});
      std::vector<size_t> pbase;
      std::vector<int> nsplit, kpers;
      size_t acc = 0;
      for (auto& side : B.L.send) {
        int M = njs * side.d, kper = 0;
        int ns = gemm_split(M, side.mul, side.D, &kper);
        pbase.push_back(acc);
        nsplit.push_back(ns);
        kpers.push_back(kper);
        acc += size_t(kDblSrcTerms) * ns * size_t(M) * side.mul * el;
      }
      int per = (njs + 7) / 8;
      for (size_t t = 0; t < terms.size(); ++t) {
        const ZTerm& T = terms[t];
        void* b[] = {(void*)&T.phi, (void*)&T.G, (void*)&gout, (void*)&d.recv, (void*)&d.src_ptr,
                     (void*)&d.src_edge, &Z, &j0, &njs, &per, &k0};
        if ((st = launch(kz, unsigned(8 * B.L.n_z_tasks * per), 64, 0, s, b, err)) != CGTP_OK) return st;
        for (size_t bi = 0; bi < B.L.send.size(); ++bi) {
          const auto& side = B.L.send[bi];
          int M = njs * side.d, Kd = side.D, kper = kpers[bi], ns = nsplit[bi];
          void* pt = xp + pbase[bi] + t * size_t(ns) * size_t(M) * side.mul * el;
          void* a[] = {&Z, (void*)&T.A, &pt, &j0, &M, &Kd, &kper};
          if ((st = launch3(kxb[bi], cdiv(M, 64), cdiv(side.mul, 64), unsigned(ns), 256, s, a, err)) != CGTP_OK)
            return st;
        }
      }
      const int nt = int(terms.size());
      for (size_t bi = 0; bi < B.L.send.size(); ++bi) {
        const auto& side = B.L.send[bi];
        int M = njs * side.d, ns = nsplit[bi] * nt;
        void* pt = xp + pbase[bi];
        void* b[] = {&pt, &ns, &M, &gg_x, &j0};
        if ((st = launch(kxr[bi], cdiv((long long)M * side.mul, 256), 256, 0, s, b, err)) != CGTP_OK) return st;
      }
    }
  }
  if (gg_pos) {
    int n = G.n;
    void* a[] = {&gev, (void*)&d.row_ptr, (void*)&d.src_ptr, (void*)&d.src_edge, &n, &gg_pos};
    if ((st = launch(kpos, unsigned(n), 64, 0, s, a, err)) != CGTP_OK) return st;
  }
  return CGTP_OK;
}

}  // namespace cgtp
