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

unsigned cdiv(long long a, long long b) { return unsigned((a + b - 1) / b); }

cgtp_status_t launch3(hipFunction_t f, unsigned gx, unsigned gy, unsigned gz, unsigned block, hipStream_t s,
                      void** args, std::string* err) {
  return launch_grid(f, gx, gy, gz, block, 0, s, args, err);
}

}  // namespace

size_t uvw_workspace(const Plan& p, const Graph& g, cgtp_op_t op) {
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

}  // namespace cgtp
