// Double backward of the channelwise convolution: the vector-Jacobian product of the backward map
// (x, r, phi, A, mbar) -> (x-bar, e-bar, phi-bar, A-bar) for cotangent directions
// (xdot, rdot, phidot, Adot) = (v_x, v_e, v_phi, v_A), following Sobek section 3.3 (Eqs. 23-31):
//   wdot = phidot A + phi Adot,  Ydot = J_Y(r) rdot,  Gdot[m1,m3] = sum_m2 c Ydot[m2],
//   Tdot = Gdot x + G xdot,  hdot = <mbar, Tdot>.
// Kernels (one family "dbl"):
//   prep2      (lane = edge):    G and Gdot rows (Ydot from a dual-number pass of the harmonics);
//   dfwd       (lane = channel): mdot_i = sum_j sum_pi (wdot T + w Tdot)         -> d/d mbar;
//   drecv      (lane = channel): A-bar-dot = sum_e phidot h + phi hdot (registers, Eq. 26) and per
//                                edge phi-bar-dot = sum Adot h + A hdot (Eq. 27), Y-bar-dot
//                                (Eq. 31) and the first-order Y-bar (Eq. 22), channel-reduced;
//   dsrc       (lane = channel): x-bar-dot_j = sum_out-edges sum_pi wdot G^T mbar + w Gdot^T mbar;
//   dedge_final(lane = edge):    e-bar-dot = J_Y^T Y-bar-dot + grad_r <J_Y(r) rdot, Y-bar> with the
//                                curvature term from nested dual numbers.
// With an in-kernel radial basis phi(|r|), phidot = phi'(|r|) (r-hat . rdot) sits in the Gdot row
// beside phi in the G row, the receiver pass adds the first-order phi-bar columns, and the edge
// finalisation adds the chain through phi and the curvature of phi to e-bar-dot.
// A missing direction is read from its primal array with a zero scale, so every load stays in
// bounds; rdot = v_edge_vec + v_pos[send] - v_pos[recv] (either part optional).
#include <algorithm>
#include <cmath>
#include <set>

#include "codegen.hpp"

namespace cgtp {

using namespace gen;

namespace {

// A and A-tangent registers per lane of one path subset in the double backward's forward-tangent
// and source passes (K values each per path).
constexpr int kDfwdRegs = 16;
// Large paths' coefficient rows are streamed in the tangent forward and the receiver pass: with
// one path per subset (forward) or per task (receiver pass) this keeps the large l <= 6 paths off
// the 256-VGPR ceiling (forward 25 %, receiver pass 33 % faster).
constexpr bool kDfwdStream = true;
constexpr int kDsrcRegs = 16;

long double dfact2(int n) {
  long double r = 1;
  for (int k = n; k > 1; k -= 2) r *= k;
  return r;
}
long double fct2(int n) {
  long double r = 1;
  for (int k = 2; k <= n; ++k) r *= k;
  return r;
}

void dual_types(Out& o) {
  // D1: value and one directional derivative.  DD: a D3 value plus epsilon times a D3 (the
  // directional derivative of a gradient-carrying value).
  o.line("struct D1 { real v, d; __device__ D1() {} __device__ D1(real c) : v(c), d(0) {}"
         " __device__ D1(real a, real b) : v(a), d(b) {} };");
  o.line("DEV D1 operator+(D1 a, D1 b) { return D1(a.v + b.v, a.d + b.d); }");
  o.line("DEV D1 operator-(D1 a, D1 b) { return D1(a.v - b.v, a.d - b.d); }");
  o.line("DEV D1 operator*(D1 a, D1 b) { return D1(a.v * b.v, a.d * b.v + a.v * b.d); }");
  o.line("DEV D1 operator*(real c, D1 b) { return D1(c * b.v, c * b.d); }");
  o.line("struct DD { D3 a, b; __device__ DD() {} __device__ DD(real c) : a(c), b(R(0)) {}"
         " __device__ DD(D3 x, D3 y) : a(x), b(y) {} };");
  o.line("DEV DD operator+(DD x, DD y) { return DD(x.a + y.a, x.b + y.b); }");
  o.line("DEV DD operator-(DD x, DD y) { return DD(x.a - y.a, x.b - y.b); }");
  o.line("DEV DD operator*(DD x, DD y) { return DD(x.a * y.a, x.a * y.b + x.b * y.a); }");
  o.line("DEV DD operator*(real c, DD y) { return DD(c * y.a, c * y.b); }");
}

// Real spherical harmonics (as in sh_eval) evaluated in type S and contracted on the fly:
// acc_k += weight_k(idx) * Y_idx for each accumulator; emitted column by column in m so that the
// Legendre intermediates die early.
void emit_sh_contract(Out& o, int L, const std::string& S, const std::string& xs, const std::string& ys,
                      const std::string& zs,
                      const std::vector<std::pair<std::string, std::function<std::string(int)>>>& accs) {
  o.open("");
  o.line(S + " a0 = " + S + "(R(1)), b0 = " + S + "(R(0));");
  o.line(S + " sx = " + xs + ", sy = " + ys + ", sz = " + zs + ";");
  for (int m = 1; m <= L; ++m)
    o.line(F("%s a%d = sx * a%d - sy * b%d, b%d = sx * b%d + sy * a%d;", S.c_str(), m, m - 1, m - 1, m, m - 1,
             m - 1));
  auto emit_y = [&](int l, int m, const std::string& q) {
    long double nrm = std::sqrt((2.0L * l + 1) * fct2(l - m) / fct2(l + m));
    if (m == 0) {
      for (auto& a : accs)
        o.line(F("%s = %s + (%s * %s) * %s;", a.first.c_str(), a.first.c_str(), a.second(l * l + l).c_str(),
                 lit(double(nrm)).c_str(), q.c_str()));
    } else {
      double c = double(nrm * std::sqrt(2.0L));
      for (auto& a : accs) {
        o.line(F("%s = %s + (%s * %s) * (%s * a%d);", a.first.c_str(), a.first.c_str(),
                 a.second(l * l + l + m).c_str(), lit(c).c_str(), q.c_str(), m));
        o.line(F("%s = %s + (%s * %s) * (%s * b%d);", a.first.c_str(), a.first.c_str(),
                 a.second(l * l + l - m).c_str(), lit(c).c_str(), q.c_str(), m));
      }
    }
  };
  for (int m = 0; m <= L; ++m) {
    o.open("");
    o.line(F("%s q%d_%d = %s(%s);", S.c_str(), m, m, S.c_str(), lit(double(dfact2(2 * m - 1))).c_str()));
    emit_y(m, m, F("q%d_%d", m, m));
    if (m + 1 <= L) {
      o.line(F("%s q%d_%d = %s * (sz * q%d_%d);", S.c_str(), m + 1, m, lit(2.0 * m + 1).c_str(), m, m));
      emit_y(m + 1, m, F("q%d_%d", m + 1, m));
    }
    for (int l = m + 2; l <= L; ++l) {
      o.line(F("%s q%d_%d = %s * (sz * q%d_%d) - %s * q%d_%d;", S.c_str(), l, m, lit(double(2 * l - 1) / (l - m)).c_str(),
               l - 1, m, lit(double(l + m - 1) / (l - m)).c_str(), l - 2, m));
      emit_y(l, m, F("q%d_%d", l, m));
    }
    o.close();
  }
  o.close();
}

// Pointers ph, phd to the current edge's K radial values and their tangent: the phi and v_phi
// inputs, or (plans with an in-kernel radial basis) the edge's G and Gdot rows (g, gd in scope).
void emit_phi_rows(Out& o, const Plan& p) {
  if (p.radial) {
    o.line(F("const real* __restrict__ ph = g + %d;", p.phi_off));
    o.line(F("const real* __restrict__ phd = gd + %d;", p.phi_off));
    return;
  }
  o.line(F("const real* __restrict__ ph = phi + (i64)e * %d;", p.K));
  o.line(F("const real* __restrict__ phd = vphi + (i64)e * %d;", p.K));
}

// Effective edge-vector direction rdot of sorted edge e (ri, sj in scope) into vex, vey, vez.
void emit_edge_direction(Out& o) {
  o.line("real vex = R(0), vey = R(0), vez = R(0);");
  o.line("if (vev) { vex = vev[3 * (i64)e]; vey = vev[3 * (i64)e + 1]; vez = vev[3 * (i64)e + 2]; }");
  o.line("if (vpos) { vex += vpos[3 * (i64)sj] - vpos[3 * (i64)ri]; vey += vpos[3 * (i64)sj + 1] - vpos[3 * (i64)ri + 1];"
         " vez += vpos[3 * (i64)sj + 2] - vpos[3 * (i64)ri + 2]; }");
}

// prep2: G (columns 0..g_stride) and Gdot (columns g_stride..2 g_stride) of every edge of [e0, e1),
// lane = edge, rows stored through the LDS tile as cgtp_prep's.
void emit_prep2(Out& o, const Plan& p) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_prep2(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ vev, const real* __restrict__ vpos, int e0,"
         " int e1, real* __restrict__ G)");
  o.line("__shared__ V4 tile[64 * 17];");
  o.line("const int lane = (int)threadIdx.x;");
  o.line("const int eb = e0 + (int)blockIdx.x * 64;");
  o.line("const int e = min(eb + lane, e1 - 1);");
  emit_edge_vector(o);
  emit_edge_direction(o);
  o.line("const real inv = R(1) / sqrt(rx * rx + ry * ry + rz * rz);");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line("const real nv = nx * vex + ny * vey + nz * vez;");
  o.line("const real dx = (vex - nx * nv) * inv, dy = (vey - ny * nv) * inv, dz = (vez - nz * nv) * inv;");
  o.line(F("D1 Y[%d];", p.sh_dim));
  o.line("sh_eval<D1>(D1(nx, dx), D1(ny, dy), D1(nz, dz), Y);");
  std::vector<std::string> vals(size_t(2 * p.g_stride), "R(0)");
  if (p.radial) {   // phi(|r|) in the G row, its tangent phi'(|r|) (r-hat . rdot) in the Gdot row
    o.line(F("real fr[%d], dfr[%d];", p.K, p.K));
    o.line("radial_eval(R(1) / inv, fr, dfr, nullptr);");
    for (int q = 0; q < p.K; ++q) {
      vals[size_t(p.phi_off + q)] = F("fr[%d]", q);
      vals[size_t(p.g_stride + p.phi_off + q)] = F("dfr[%d] * nv", q);
    }
  }
  for (const Path& P : p.paths) {
    int s = P.l2 * P.l2;
    int n = P.g_off;
    for (const GPair& gp : P.gpairs) {
      std::string ev, ed;
      for (auto& t : gp.terms) {
        if (!ev.empty()) {
          ev += " + ";
          ed += " + ";
        }
        ev += lit(t.second) + " * Y[" + std::to_string(s + t.first) + "].v";
        ed += lit(t.second) + " * Y[" + std::to_string(s + t.first) + "].d";
      }
      vals[size_t(n)] = ev;
      vals[size_t(n + p.g_stride)] = ed;
      ++n;
    }
  }
  emit_staged_rows(o, p, vals, 2 * p.g_stride);
  o.close();
}

const char* kDArgs =
    "const real* __restrict__ x, const real* __restrict__ vx, const real* __restrict__ phi,"
    " const real* __restrict__ vphi, const real* __restrict__ A, const real* __restrict__ vA,"
    " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
    " const real* __restrict__ gout, real* __restrict__ out, real* __restrict__ ep, real* __restrict__ ap,"
    " real sx, real sphi, real sA";

// Edge loop over the receiver's in-edges (one wave); loads x and xdot rows, phi and phidot, the G
// and Gdot rows.  Body sees e, g (G row), gd (Gdot row), f<q>, fd<q>, x<b>_<m>, xd<b>_<m>.
// nE > 1 (2 or 4): lane group h_ (64 / nE lanes, `h_` in scope) takes edge eb + h_ of each step
// of nE edges; e, j and the row pointers are then per lane, and a group past the last edge reads
// the step's first edge with zero phi and phi-dot (`ok_` false; the values are loaded
// unconditionally and masked, since a load under the condition becomes a branch per value).
void emit_dedge_loop(Out& o, const Plan& p, const std::vector<int>& blocks, const std::function<void()>& body,
                     int nE = 1) {
  if (nE > 1) {
    o.open(F("for (int eb_ = e0; eb_ < e1; eb_ += %d)", nE));
    o.line("const bool ok_ = eb_ + h_ < e1;");
    o.line("const int e = ok_ ? eb_ + h_ : eb_;");
  } else {
    o.open("for (int e = e0; e < e1; ++e)");
    o.line("const bool ok_ = true;");
  }
  o.line("const int j = col[e];");
  o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", 2 * p.g_stride));
  o.line(F("const real* __restrict__ gd = g + %d;", p.g_stride));
  emit_phi_rows(o, p);
  for (int q = 0; q < p.K; ++q)
    o.line(F("const real fl%d_ = ph[%d], fdl%d_ = phd[%d];", q, q, q, q) +
           F(" const real f%d = ok_ ? fl%d_ : R(0), fd%d = ok_ ? sphi * fdl%d_ : R(0);", q, q, q, q));
  for (int b : blocks) {
    const Block& B = p.in[b];
    for (int m = 0; m < B.dim(); ++m) {
      o.line(F("const real x%d_%d = x[(i64)j * %d + %d + uc];", b, m, p.c_in, B.offset + m * B.mul));
      o.line(F("const real xd%d_%d = sx * vx[(i64)j * %d + %d + uc];", b, m, p.c_in, B.offset + m * B.mul));
    }
  }
  body();
  o.close();
}

void emit_da_loads(Out& o, const Plan& p, const std::vector<int>& paths) {
  for (int pi : paths) {
    const Path& P = p.paths[pi];
    for (int q = 0; q < p.K; ++q) {
      o.line(F("const real a%d_%d = A[%d + uc];", pi, q, q * p.n_w + P.w_off));
      o.line(F("const real ad%d_%d = sA * vA[%d + uc];", pi, q, q * p.n_w + P.w_off));
    }
  }
}

// w and wdot of path pi.
void emit_wwd(Out& o, const Plan& p, int pi) {
  o.line(F("real w%d = f0 * a%d_0;", pi, pi));
  o.line(F("real wd%d = fma(fd0, a%d_0, f0 * ad%d_0);", pi, pi, pi));
  for (int q = 1; q < p.K; ++q) {
    o.line(F("w%d = fma(f%d, a%d_%d, w%d);", pi, q, pi, q, pi));
    o.line(F("wd%d = fma(fd%d, a%d_%d, fma(f%d, ad%d_%d, wd%d));", pi, q, pi, q, q, pi, q, pi));
  }
}

// T[m3] = G x and Tdot[m3] = Gdot x + G xdot of path pi, names t<pi>_<m3>, td<pi>_<m3>.  With
// `rc` the G and Gdot coefficients come by row broadcast from the chunks rc[0] (G) and rc[1] (Gdot).
std::vector<bool> emit_t_td(Out& o, const Plan& p, int pi, int d3, bool stream, RowChunks* rc = nullptr) {
  const Path& P = p.paths[pi];
  std::vector<bool> started(d3, false);
  if (rc) {
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      const int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3, idx = P.g_off + int(t);
      const bool first = !started[m3];
      o.line(bcast_term(o, rc[0], idx, F("t%d_%d", pi, m3), F("x%d_%d", P.i_in, m1), first));
      o.line(bcast_term(o, rc[0], idx, F("td%d_%d", pi, m3), F("xd%d_%d", P.i_in, m1), first));
      o.line(bcast_term(o, rc[1], idx, F("td%d_%d", pi, m3), F("x%d_%d", P.i_in, m1), false));
      started[m3] = true;
    }
    return started;
  }
  GStream gs(o, p, pi, "g", "", stream), gds(o, p, pi, "gd", "d", stream);
  for (size_t t = 0; t < P.gpairs.size(); ++t) {
    int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
    const std::string G = gs.ref(int(t)), Gd = gds.ref(int(t));
    if (!started[m3]) {
      o.line(F("real t%d_%d = %s * x%d_%d;", pi, m3, G.c_str(), P.i_in, m1));
      o.line(F("real td%d_%d = fma(%s, x%d_%d, %s * xd%d_%d);", pi, m3, Gd.c_str(), P.i_in, m1, G.c_str(), P.i_in,
               m1));
    } else {
      o.line(F("t%d_%d = fma(%s, x%d_%d, t%d_%d);", pi, m3, G.c_str(), P.i_in, m1, pi, m3));
      o.line(F("td%d_%d = fma(%s, x%d_%d, fma(%s, xd%d_%d, td%d_%d));", pi, m3, Gd.c_str(), P.i_in, m1, G.c_str(),
               P.i_in, m1, pi, m3));
    }
    started[m3] = true;
  }
  return started;
}

// mdot of task (output block k, channel block) for one receiver (Eq. 25).
void emit_dfwd_task(Out& o, const Plan& p, int ti, const Task& T) {
  const Block& OB = p.out[T.group];
  const int d3 = OB.dim(), MUL = OB.mul;
  // Blocks of at most 32 channels in fp32: 2 or 4 edges per wave step, one per lane group, with
  // the G and Gdot coefficients by row broadcast; the groups' partial sums are added at the end.
  const int nE = bcast_edges_per_wave(p, MUL), gsz = 64 / nE;
  const bool bcast = nE > 1 && p.dtype != CGTP_F64;
  o.open(F("DEV void dfw_t%d(%s, int node, int e_base)", ti, kDArgs));
  emit_vz(o, p);
  o.line("const int lane = (int)threadIdx.x & 63;");
  if (nE > 1) {
    o.line(F("const int u = lane %% %d, h_ = lane / %d;", gsz, gsz));
    if (bcast) o.line("const int r16_ = lane & 15;");
  } else {
    o.line(F("const int u = %d + lane;", T.cb * 64));
  }
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d3; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  for (const auto& S : a_subsets(p, T.paths, kDfwdRegs)) {  // A and its tangent
    o.open("");
    emit_da_loads(o, p, S);
    emit_dedge_loop(o, p, in_blocks_of(p, S), [&] {
      const auto order = chunks_of(g_ranges(p, S));
      RowChunks rc[2] = {{p.g_stride, "g", "", order}, {p.g_stride, "gd", "d", order}};
      for (int pi : S) {
        emit_wwd(o, p, pi);
        auto started = emit_t_td(o, p, pi, d3, kDfwdStream, bcast ? rc : nullptr);
        for (int m = 0; m < d3; ++m)
          if (started[m]) o.line(F("acc%d = fma(wd%d, t%d_%d, fma(w%d, td%d_%d, acc%d));", m, pi, pi, m, pi, pi, m, m));
      }
    }, nE);
    o.close();
  }
  for (int span = gsz; span < 64; span *= 2)
    for (int m = 0; m < d3; ++m) o.line(F("acc%d += __shfl_xor(acc%d, %d);", m, m, span));
  o.open(nE > 1 ? F("if (lane < %d && u < %d)", gsz, MUL) : F("if (u < %d)", MUL));
  o.line(F("real* __restrict__ dst = out + (i64)node * %d + %d + u;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("dst[%d] = acc%d;", m * MUL, m));
  o.close();
  o.close();
}

// Receiver-major part of task (output block k, path subset, channel block) for one receiver per wave.
// Edge partial columns of the task: [0, K) phi-bar-dot, [K, K+Yd) Y-bar-dot, [K+Yd, K+2Yd) Y-bar.
void emit_drecv_task(Out& o, const Plan& p, int ti, const Task& T, int col_off, int row) {
  const Block& OB = p.out[T.group];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  const std::vector<int> yc = recv_task_ycols(p, T);
  const int ny = int(yc.size()), V = dbl_task_width(p, T);
  // Columns: K phi-bar-dot partials, then Y-bar-dot and first-order Y-bar over the task's Y entries.
  auto cd = [&](int y) { return K + int(std::find(yc.begin(), yc.end(), y) - yc.begin()); };
  auto cw = [&](int y) { return cd(y) + ny; };
  // With an in-kernel radial basis, K more columns: the first-order phi-bar (A h) of the task,
  // for the curvature of phi(|r|) in the edge-vector gradient.
  auto cb = [&](int q) { return K + 2 * ny + q; };
  // Blocks of at most 16 channels: 4 edges per wave step.  In fp64, 32-channel blocks keep one
  // edge per step (two measured slower: per-lane coefficient rows of G and G-dot cost the
  // registers that the wave-uniform rows keep in scalar ones); in fp32 the coefficients come by
  // row broadcast and 32-channel blocks take 2 edges per step.
  const bool f64 = p.dtype == CGTP_F64;
  const int nE = f64 ? (MUL <= 16 ? 4 : 1) : bcast_edges_per_wave(p, MUL), gsz = 64 / nE;
  const bool bcast = nE > 1 && !f64;
  o.open(F("DEV void drc_t%d(%s, real* sm, int node, int e_base, int eps, int slot)", ti, kDArgs));
  emit_vz(o, p);
  o.line("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  if (bcast) o.line("const int r16_ = lane & 15;");
  if (nE > 1)
    o.line(F("const int u = lane %% %d, h_ = lane / %d;", gsz, gsz));
  else
    o.line(F("const int u = %d + lane;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  emit_da_loads(o, p, T.paths);
  int na = 0;
  for (size_t k = 0; k < T.paths.size() * size_t(K); ++k) o.line(F("real aa%d = R(0);", na++));
  o.open("if (node >= 0)");
  o.line(F("const real* __restrict__ gr = gout + (i64)node * %d + %d + uc;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("const real mb%d = u < %d ? gr[%d] : R(0);", m, MUL, m * MUL));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  emit_dedge_loop(o, p, in_blocks_of(p, T.paths), [&] {
    for (int v = 0; v < V; ++v) o.line(F("real v%d = R(0);", v));
    int ai = 0;
    const auto order = chunks_of(g_ranges(p, T.paths));
    RowChunks rc[2] = {{p.g_stride, "g", "", order}, {p.g_stride, "gd", "d", order}};
    for (int pi : T.paths) {
      const Path& P = p.paths[pi];
      const int y0 = P.l2 * P.l2;
      emit_wwd(o, p, pi);
      auto started = emit_t_td(o, p, pi, d3, kDfwdStream, bcast ? rc : nullptr);
      bool first = true;
      for (int m = 0; m < d3; ++m)
        if (started[m]) {
          if (first) {
            o.line(F("real h%d = mb%d * t%d_%d;", pi, m, pi, m));
            o.line(F("real hd%d = mb%d * td%d_%d;", pi, m, pi, m));
          } else {
            o.line(F("h%d = fma(mb%d, t%d_%d, h%d);", pi, m, pi, m, pi));
            o.line(F("hd%d = fma(mb%d, td%d_%d, hd%d);", pi, m, pi, m, pi));
          }
          first = false;
        }
      for (int q = 0; q < K; ++q, ++ai) {
        o.line(F("aa%d = fma(fd%d, h%d, fma(f%d, hd%d, aa%d));", ai, q, pi, q, pi, ai));
        o.line(F("v%d = fma(ad%d_%d, h%d, fma(a%d_%d, hd%d, v%d));", q, pi, q, pi, pi, q, pi, q));
        if (p.radial) o.line(F("v%d = fma(a%d_%d, h%d, v%d);", cb(q), pi, q, pi, cb(q)));
      }
      const int d1 = 2 * P.l1 + 1;
      for (int m = 0; m < d1; ++m)
        o.line(F("const real s%d_%d = fma(wd%d, x%d_%d, w%d * xd%d_%d);", pi, m, pi, P.i_in, m, pi, P.i_in, m));
      std::set<int> m3used;
      for (auto& gp : P.gpairs) m3used.insert(gp.m3);
      for (int m : m3used) o.line(F("const real wm%d_%d = w%d * mb%d;", pi, m, pi, m));
      for (auto& gp : P.gpairs) {
        o.line(F("{ const real z = s%d_%d * mb%d, zw = x%d_%d * wm%d_%d;", pi, gp.m1, gp.m3, P.i_in, gp.m1, pi, gp.m3));
        for (auto& t : gp.terms) {
          o.line(F("  v%d = fma(%s, z, v%d);", cd(y0 + t.first), lit(t.second).c_str(), cd(y0 + t.first)));
          o.line(F("  v%d = fma(%s, zw, v%d);", cw(y0 + t.first), lit(t.second).c_str(), cw(y0 + t.first)));
        }
        o.line("}");
      }
    }
    if (nE > 1) {   // one edge per group: its columns reduced over the group's lanes and stored
      emit_group_reduce_store(o, V, (p.radial ? 2 : 1) * K + 2 * ny, gsz, p.dtype == CGTP_F64,
                              F("ep + ((i64)((e - e_base) >> 6) * %d + %d) * 64 + ((e - e_base) & 63)", row, col_off));
      return;
    }
    const int H = V / 2, Q = V / 4;
    std::vector<std::pair<std::string, std::string>> pr;
    for (int k = 0; k < H; ++k) pr.push_back({F("v%d", k), F("v%d", k + H)});
    emit_swaps(o, pr, 32, f64);
    for (int k = 0; k < H; ++k) o.line(F("v%d += v%d;", k, k + H));
    pr.clear();
    for (int k = 0; k < Q; ++k) pr.push_back({F("v%d", k), F("v%d", k + Q)});
    emit_swaps(o, pr, 16, f64);
    for (int k = 0; k < Q; ++k) o.line(F("v%d += v%d;", k, k + Q));
    if (!f64) {   // column r Q + k of row r in v_k
      emit_row_reduce_store(o, Q, "true", [&](const std::string& kk, const std::string& val) {
        return F("ep[((i64)((e - e_base) >> 6) * %d + %d + r_ * %d + ", row, col_off, Q) + kk +
               ") * 64 + ((e - e_base) & 63)] = " + val + ";";
      });
      return;
    }
    for (int k = 0; k < Q; ++k) o.line(F("v%d = rowsum(v%d); asm volatile(\"\" : \"+v\"(v%d));", k, k, k));
    o.open("if ((lane & 15) == 0)");
    o.line(F("real* __restrict__ dst = ep + ((i64)((e - e_base) >> 6) * %d + %d + (lane >> 4) * %d) * 64"
             " + ((e - e_base) & 63);", row, col_off, Q));
    for (int k = 0; k < Q; ++k) o.line(F("dst[%d] = v%d;", 64 * k, k));
    o.close();
  }, nE);
  for (int span = gsz; span < 64; span *= 2)
    for (int k = 0; k < na; ++k) o.line(F("aa%d += __shfl_xor(aa%d, %d);", k, k, span));
  o.close();
  emit_wave_combine(o, "aa", na, 4);
  o.open(nE > 1 ? F("if (w == 0 && lane < %d && u < %d)", gsz, MUL) : F("if (w == 0 && u < %d)", MUL));
  o.line(F("real* __restrict__ dst = ap + (i64)slot * %d + u;", K * p.n_w));
  int ai = 0;
  for (int pi : T.paths)
    for (int q = 0; q < K; ++q, ++ai) o.line(F("dst[%d] += aa%d;", q * p.n_w + p.paths[pi].w_off, ai));
  o.close();
  o.close();
}

const char* kDSrcArgs =
    "const real* __restrict__ phi, const real* __restrict__ vphi, const real* __restrict__ A,"
    " const real* __restrict__ vA, const real* __restrict__ G, const real* __restrict__ gout,"
    " const int* __restrict__ recv, const int* __restrict__ src_beg, const int* __restrict__ src_end,"
    " const int* __restrict__ src_edge,"
    " real* __restrict__ gx, real sphi, real sA";

// x-bar-dot of task (input block b, channel block) for one sender (Eq. 30).
void emit_dsrc_task(Out& o, const Plan& p, int ti, const Task& T) {
  const Block& IB = p.in[T.group];
  const int d1 = IB.dim(), MUL = IB.mul, K = p.K;
  // Blocks of at most 32 channels in fp32: 2 or 4 out-edges per wave step, one per lane group,
  // with the G and Gdot coefficients by row broadcast; the groups' partial sums are added at the end.
  const int nE = bcast_edges_per_wave(p, MUL), gsz = 64 / nE;
  const bool bcast = nE > 1 && p.dtype != CGTP_F64;
  o.open(F("DEV void dsr_t%d(%s, int node, int e_base, int accumulate)", ti, kDSrcArgs));
  emit_vz(o, p);
  o.line("const int lane = (int)threadIdx.x & 63;");
  if (nE > 1) {
    o.line(F("const int u = lane %% %d, h_ = lane / %d;", gsz, gsz));
    if (bcast) o.line("const int r16_ = lane & 15;");
  } else {
    o.line(F("const int u = %d + lane;", T.cb * 64));
  }
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d1; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int s0 = src_beg[node], s1 = src_end[node];");
  for (const auto& S : a_subsets(p, T.paths, kDsrcRegs)) {
    o.open("");
    emit_da_loads(o, p, S);
    // Edge ids and receivers of up to 64 out-edges, one per lane, taken with readlane (one
    // edge per step) or, per lane group, with a lane shuffle (nE edges per step; el_ and il_ hold
    // valid ids in every lane, and a group past the last edge gets zero phi and phi-dot).
    o.open("for (int kb_ = s0; kb_ < s1; kb_ += 64)");
    o.line("const int kl_ = kb_ + lane;");
    o.line("const int el_ = src_edge[kl_ < s1 ? kl_ : kb_];");
    o.line("const int il_ = recv[el_];");
    o.line("const int ne_ = min(64, s1 - kb_);");
    if (nE > 1) {
      o.open(F("for (int k_ = 0; k_ < ne_; k_ += %d)", nE));
      o.line("const bool ok_ = k_ + h_ < ne_;");
      o.line("const int e = __shfl(el_, k_ + h_);");
      o.line("const int i = __shfl(il_, k_ + h_);");
    } else {
      o.open("for (int k_ = 0; k_ < ne_; ++k_)");
      o.line("const bool ok_ = true;");
      o.line("const int e = __builtin_amdgcn_readlane(el_, k_);");
      o.line("const int i = __builtin_amdgcn_readlane(il_, k_);");
    }
    o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", 2 * p.g_stride));
    o.line(F("const real* __restrict__ gd = g + %d;", p.g_stride));
    emit_phi_rows(o, p);
    for (int q = 0; q < K; ++q)
      o.line(F("const real fl%d_ = ph[%d], fdl%d_ = phd[%d];", q, q, q, q) +
             F(" const real f%d = ok_ ? fl%d_ : R(0), fd%d = ok_ ? sphi * fdl%d_ : R(0);", q, q, q, q));
    o.line(F("const real* __restrict__ gi = gout + (i64)i * %d + uc;", p.c_out));
    for (int ob : out_blocks_of(p, S)) {
      const Block& B = p.out[ob];
      for (int m = 0; m < B.dim(); ++m) o.line(F("const real mb%d_%d = gi[%d];", ob, m, B.offset + m * B.mul));
    }
    const auto order = chunks_of(g_ranges(p, S));
    RowChunks rc[2] = {{p.g_stride, "g", "", order}, {p.g_stride, "gd", "d", order}};
    for (int pi : S) {
      const Path& P = p.paths[pi];
      emit_wwd(o, p, pi);
      std::vector<bool> started(d1, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (bcast) {
          const int idx = P.g_off + int(t);
          o.line(bcast_term(o, rc[0], idx, F("b%d_%d", pi, m1), F("mb%d_%d", P.i_out, m3), !started[m1]));
          o.line(bcast_term(o, rc[1], idx, F("bd%d_%d", pi, m1), F("mb%d_%d", P.i_out, m3), !started[m1]));
          started[m1] = true;
          continue;
        }
        const std::string G = gref(p, pi, int(t), "g", "", false), Gd = gref(p, pi, int(t), "gd", "d", false);
        if (!started[m1]) {
          o.line(F("real b%d_%d = %s * mb%d_%d;", pi, m1, G.c_str(), P.i_out, m3));
          o.line(F("real bd%d_%d = %s * mb%d_%d;", pi, m1, Gd.c_str(), P.i_out, m3));
        } else {
          o.line(F("b%d_%d = fma(%s, mb%d_%d, b%d_%d);", pi, m1, G.c_str(), P.i_out, m3, pi, m1));
          o.line(F("bd%d_%d = fma(%s, mb%d_%d, bd%d_%d);", pi, m1, Gd.c_str(), P.i_out, m3, pi, m1));
        }
        started[m1] = true;
      }
      for (int m = 0; m < d1; ++m)
        if (started[m]) o.line(F("acc%d = fma(wd%d, b%d_%d, fma(w%d, bd%d_%d, acc%d));", m, pi, pi, m, pi, pi, m, m));
    }
    o.close();
    o.close();
    o.close();
  }
  for (int span = gsz; span < 64; span *= 2)
    for (int m = 0; m < d1; ++m) o.line(F("acc%d += __shfl_xor(acc%d, %d);", m, m, span));
  o.open(nE > 1 ? F("if (lane < %d && u < %d)", gsz, MUL) : F("if (u < %d)", MUL));
  o.line(F("real* __restrict__ dst = gx + (i64)node * %d + %d + u;", p.c_in, IB.offset));
  o.open("if (accumulate)");
  for (int m = 0; m < d1; ++m) o.line(F("dst[%d] += acc%d;", m * MUL, m));
  o.close("} else {");
  ++o.ind;
  for (int m = 0; m < d1; ++m) o.line(F("dst[%d] = acc%d;", m * MUL, m));
  o.close();
  o.close();
  o.close();
}

// e-bar-dot of edge e (lane = edge) from Y-bar-dot ybd[] and the first-order Y-bar ybw[], which
// `fill` assigns: J_Y^T ybd + grad_r <J_Y(r) rdot, ybw>, into gx, gy, gz.  Also leaves in scope
// the unit vector nx, ny, nz, inv = 1 / |r|, the direction rdot (vex, vey, vez) and nv = n . rdot.
void emit_ebar_dot(Out& o, const Plan& p, const std::function<void()>& fill) {
  const int Yd = p.sh_dim;
  emit_edge_vector(o);
  emit_edge_direction(o);
  o.line("const real inv = R(1) / sqrt(rx * rx + ry * ry + rz * rz);");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line("const real nv = nx * vex + ny * vey + nz * vez;");
  o.line("const real dx = (vex - nx * nv) * inv, dy = (vey - ny * nv) * inv, dz = (vez - nz * nv) * inv;");
  o.line(F("real ybd[%d], ybw[%d];", Yd, Yd));
  fill();
  o.line("DD accw(R(0));");
  o.line("DD accd(R(0));");
  emit_sh_contract(o, p.lmax, "DD", "DD(D3(nx, R(1), R(0), R(0)), D3(dx, R(0), R(0), R(0)))",
                   "DD(D3(ny, R(0), R(1), R(0)), D3(dy, R(0), R(0), R(0)))",
                   "DD(D3(nz, R(0), R(0), R(1)), D3(dz, R(0), R(0), R(0)))",
                   {{"accw", [](int i) { return F("ybw[%d]", i); }}, {"accd", [](int i) { return F("ybd[%d]", i); }}});
  // J^T Ybar_d = Pi p_d / rho with p_d the gradient of sum Ybar_d P at n.
  o.line("real px = accd.a.x, py = accd.a.y, pz = accd.a.z;");
  o.line("real pn = nx * px + ny * py + nz * pz;");
  o.line("real gx = (px - nx * pn) * inv, gy = (py - ny * pn) * inv, gz = (pz - nz * pn) * inv;");
  // Curvature: H v = [-dn (n.p) - n (dn.p) + Pi (H_P dn)] / rho - Pi p (n.v) / rho^2, p, H_P dn of sum Ybar_w P.
  o.line("const real wx = accw.a.x, wy = accw.a.y, wz = accw.a.z;");
  o.line("const real hx = accw.b.x, hy = accw.b.y, hz = accw.b.z;");
  o.line("const real np_ = nx * wx + ny * wy + nz * wz, dp = dx * wx + dy * wy + dz * wz;");
  o.line("const real nh = nx * hx + ny * hy + nz * hz;");
  o.line("gx += (-dx * np_ - nx * dp + (hx - nx * nh)) * inv - (wx - nx * np_) * nv * inv * inv;");
  o.line("gy += (-dy * np_ - ny * dp + (hy - ny * nh)) * inv - (wy - ny * np_) * nv * inv * inv;");
  o.line("gz += (-dz * np_ - nz * dp + (hz - nz * nh)) * inv - (wz - nz * np_) * nv * inv * inv;");
}

// Gdot row (G's layout) of the current edge e, stored through the LDS tile (lane = edge; `tile`,
// `lane`, `eb`, `e0`, `e1` and the destination `G` in scope): the directional derivative of G
// along rdot, from a dual-number pass of the harmonics.
void emit_gdot_row(Out& o, const Plan& p) {
  emit_edge_vector(o);
  emit_edge_direction(o);
  o.line("const real inv = R(1) / sqrt(rx * rx + ry * ry + rz * rz);");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line("const real nv = nx * vex + ny * vey + nz * vez;");
  o.line("const real dx = (vex - nx * nv) * inv, dy = (vey - ny * nv) * inv, dz = (vez - nz * nv) * inv;");
  o.line(F("D1 Y[%d];", p.sh_dim));
  o.line("sh_eval<D1>(D1(nx, dx), D1(ny, dy), D1(nz, dz), Y);");
  std::vector<std::string> vals(size_t(p.g_stride), "R(0)");
  for (const Path& P : p.paths) {
    int s = P.l2 * P.l2;
    int n = P.g_off;
    for (const GPair& gp : P.gpairs) {
      std::string ed;
      for (auto& t : gp.terms) {
        if (!ed.empty()) ed += " + ";
        ed += lit(t.second) + " * Y[" + std::to_string(s + t.first) + "].d";
      }
      vals[size_t(n++)] = ed;
    }
  }
  emit_staged_rows(o, p, vals, p.g_stride);
}

// Edge finalisation: phi-bar-dot sums, e-bar-dot = J^T Ybar_d + the curvature term.
void emit_dedge_final(Out& o, const Plan& p, const std::vector<Task>& tasks) {
  const int K = p.K, Yd = p.sh_dim, row = dbl_partial_row(p);
  std::vector<int> off;
  std::vector<std::vector<int>> yc;
  for (int k = 0, c = 0; k < int(tasks.size()); c += dbl_task_width(p, tasks[k]), ++k) {
    off.push_back(c);
    yc.push_back(recv_task_ycols(p, tasks[k]));
  }
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_dedge_final(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ vev, const real* __restrict__ vpos,"
         " const real* __restrict__ ep, int e0, int e1, int eps, real* __restrict__ gphi, real* __restrict__ gev)");
  o.line("const int e = e0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  o.line("(void)eps;");
  o.line(F("const real* __restrict__ rw = ep + (i64)((e - e0) >> 6) * %d + ((e - e0) & 63);", 64 * row));
  o.line("#define ROWV(k) rw[64 * (k)]");
  // Sum of one kind of column over the tasks in order; `shift` 0: Y-bar-dot, 1: first-order Y-bar.
  auto sum_y = [&](int y, int shift) {
    std::string ex;
    for (size_t t = 0; t < tasks.size(); ++t) {
      auto it = std::find(yc[t].begin(), yc[t].end(), y);
      if (it == yc[t].end()) continue;
      const int c = off[t] + K + int(it - yc[t].begin()) + shift * int(yc[t].size());
      ex += (ex.empty() ? "" : " + ") + F("ROWV(%d)", c);
    }
    return ex.empty() ? std::string("R(0)") : ex;
  };
  for (int q = 0; q < K; ++q) {
    std::string ex;
    for (size_t t = 0; t < tasks.size(); ++t) ex += (t ? " + " : "") + F("ROWV(%d)", off[t] + q);
    o.line(F("const real gp%d = ", q) + ex + ";");
  }
  o.open("if (gphi)");
  for (int q = 0; q < K; ++q) o.line(F("gphi[(i64)e * %d + %d] = gp%d;", K, q, q));
  o.close();
  o.line("if (!gev) return;");
  emit_ebar_dot(o, p, [&] {
    for (int m = 0; m < Yd; ++m) {
      o.line(F("ybd[%d] = ", m) + sum_y(m, 0) + ";");
      o.line(F("ybw[%d] = ", m) + sum_y(m, 1) + ";");
    }
  });
  if (p.radial) {
    // Through phi(|r|): the chain J_phi^T phi-bar-dot = (sum gp phi') r-hat, and the curvature
    // grad_r [s (r-hat . rdot)] = s' t r-hat + s (rdot - t r-hat) / |r| with s = sum phi-bar phi',
    // s' = sum phi-bar phi'', t = r-hat . rdot.
    for (int q = 0; q < K; ++q) {
      std::string ex;
      for (size_t t = 0; t < tasks.size(); ++t)
        ex += (t ? " + " : "") + F("ROWV(%d)", off[t] + K + 2 * int(yc[t].size()) + q);
      o.line(F("const real pb%d = ", q) + ex + ";");
    }
    o.line(F("real fr[%d], dfr[%d], d2fr[%d];", K, K, K));
    o.line("radial_eval(R(1) / inv, fr, dfr, d2fr);");
    o.line("real sc = R(0), s1 = R(0), s2 = R(0);");
    for (int q = 0; q < K; ++q) {
      o.line(F("sc = fma(gp%d, dfr[%d], sc);", q, q));
      o.line(F("s1 = fma(pb%d, dfr[%d], s1);", q, q));
      o.line(F("s2 = fma(pb%d, d2fr[%d], s2);", q, q));
    }
    o.line("const real cn = sc + (s2 - s1 * inv) * nv, cv = s1 * inv;");
    o.line("gx += cn * nx + cv * vex; gy += cn * ny + cv * vey; gz += cn * nz + cv * vez;");
  }
  o.line("gev[3 * (i64)e] = gx; gev[3 * (i64)e + 1] = gy; gev[3 * (i64)e + 2] = gz;");
  o.line("#undef ROWV");
  o.close();
}

}  // namespace

int dbl_task_width(const Plan& p, const Task& T) {
  return ((p.radial ? 2 : 1) * p.K + 2 * int(recv_task_ycols(p, T).size()) + 3) / 4 * 4;
}

int dbl_partial_row(const Plan& p) { return task_tables(p).dbl_row; }

std::string generate_dbl_source(const Plan& p, std::string* err) {
  if (p.mode != CGTP_CHANNELWISE) {
    *err = "the double backward is generated for the channelwise mode";
    return "";
  }
  Out o;
  prelude(o, p, true, true);
  dual_types(o);
  emit_sh(o, p.lmax);
  emit_prep2(o, p);
  auto ft = forward_tasks(p);
  for (int k = 0; k < int(ft.size()); ++k) emit_dfwd_task(o, p, k, ft[k]);
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  // order (nullable): slot -> node of a launch over every node, heaviest first per XCD range.
  o.open(std::string("cgtp_dfwd(") + kDArgs + ", int i0, int nrec, int per, int e_base, const int* __restrict__ order)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, i = xcd * per + (s - t * per);");
  o.line("if (i >= nrec) return;");
  o.line("const int node = order ? order[i] : i0 + i;");
  o.open("switch (t)");
  for (int k = 0; k < int(ft.size()); ++k)
    o.line(F("case %d: dfw_t%d(x, vx, phi, vphi, A, vA, G, row_ptr, col, gout, out, ep, ap, sx, sphi, sA, node, e_base);"
             " break;", k, k));
  o.line("default: break;");
  o.close();
  o.close();
  auto rt = dbl_recv_tasks(p);
  const int row = dbl_partial_row(p);
  int amax = 0;
  for (int k = 0, off = 0; k < int(rt.size()); off += dbl_task_width(p, rt[k]), ++k) {
    emit_drecv_task(o, p, k, rt[k], off, row);
    amax = std::max(amax, int(rt[k].paths.size()) * p.K);
  }
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open(std::string("cgtp_drecv(") + kDArgs +
         ", int i0, int nrec, int per, int nch, int e_base, int eps, const int* __restrict__ order)");
  o.line(F("__shared__ real sm[%d];", 3 * amax * 64));
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / nch, c = s - t * nch;");
  o.line("const int lo = xcd * per + c * 4;");
  o.line("int hi = lo + 4; if (hi > (xcd + 1) * per) hi = (xcd + 1) * per; if (hi > nrec) hi = nrec;");
  o.line("if (lo >= hi) return;");
  o.line("const int r = lo + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  o.line("const int node = r < hi ? (order ? order[r] : i0 + r) : -1;");
  o.line("const int slot = xcd * nch + c;");
  o.open("switch (t)");
  for (int k = 0; k < int(rt.size()); ++k)
    o.line(F("case %d: drc_t%d(x, vx, phi, vphi, A, vA, G, row_ptr, col, gout, out, ep, ap, sx, sphi, sA, sm, node,"
             " e_base, eps, slot); break;", k, k));
  o.line("default: break;");
  o.close();
  o.close();
  auto st = source_tasks(p);
  for (int k = 0; k < int(st.size()); ++k) emit_dsrc_task(o, p, k, st[k]);
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open(std::string("cgtp_dsrc(") + kDSrcArgs +
         ", int nrec, int per, int e_base, int accumulate, const int* __restrict__ order)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, slot = xcd * per + (s - t * per);");
  o.line("if (slot >= nrec) return;");
  o.line("const int node = order ? order[slot] : slot;");
  o.open("switch (t)");
  for (int k = 0; k < int(st.size()); ++k)
    o.line(F("case %d: dsr_t%d(phi, vphi, A, vA, G, gout, recv, src_beg, src_end, src_edge, gx, sphi, sA, node, e_base,"
             " accumulate); break;", k, k));
  o.line("default: break;");
  o.close();
  o.close();
  emit_dedge_final(o, p, rt);
  emit_small_kernels(o);
  return o.s.str();
}

namespace gen {

// Kernels of the fully connected double backward beyond the first-order passes it reuses:
//   cgtp_prep_dot / cgtp_prep_src_dot: Gdot rows of the edges of a receiver chunk (receiver
//     order) or of a sender chunk (source-CSR order), the tangent of G along rdot;
//   cgtp_uvw_dedge_final: phi-bar-dot and e-bar-dot of each edge from the partial columns of up
//     to three edge passes (their sums are phi-bar-dot and Y-bar-dot) and of the first-order pass
//     (Y-bar, for the curvature term); each buffer holds ntask tasks of V columns, K phi-bar
//     columns then sh_dim Y-bar columns, column c of edge e at c eps + (e - e0).
void emit_uvw_dbl_kernels(Out& o, const Plan& p, int ntask, int V) {
  const int K = p.K, Yd = p.sh_dim;
  dual_types(o);
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_prep_dot(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ vev, const real* __restrict__ vpos, int e0,"
         " int e1, real* __restrict__ Gd)");
  o.line("__shared__ V4 tile[64 * 17];");
  o.line("real* __restrict__ G = Gd;");
  o.line("const int lane = (int)threadIdx.x;");
  o.line("const int eb = e0 + (int)blockIdx.x * 64;");
  o.line("const int e = min(eb + lane, e1 - 1);");
  emit_gdot_row(o, p);
  o.close();
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_prep_src_dot(const real* __restrict__ pos, const real* __restrict__ shift,"
         " const int* __restrict__ recv, const int* __restrict__ send, const int* __restrict__ src_edge,"
         " const real* __restrict__ vev, const real* __restrict__ vpos, int k0, int k1, real* __restrict__ Gd)");
  // Rows at source-CSR positions: the staged stores index them by k (eb, e0, e1 name positions).
  o.line("__shared__ V4 tile[64 * 17];");
  o.line("real* __restrict__ G = Gd;");
  o.line("const int lane = (int)threadIdx.x;");
  o.line("const int e0 = k0, e1 = k1, eb = k0 + (int)blockIdx.x * 64;");
  o.line("const int e = src_edge[min(eb + lane, k1 - 1)];");
  emit_gdot_row(o, p);
  o.close();
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_uvw_dedge_final(const real* __restrict__ pos, const real* __restrict__ shift,"
         " const int* __restrict__ recv, const int* __restrict__ send, const real* __restrict__ vev,"
         " const real* __restrict__ vpos, const real* __restrict__ epa, const real* __restrict__ epb,"
         " const real* __restrict__ epc, const real* __restrict__ epw, int e0, int e1, int eps,"
         " real* __restrict__ gphi, real* __restrict__ gev, real* __restrict__ pb1)");
  o.line("const int e = e0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  o.line("const i64 el_ = e - e0;");
  // Column c summed over the tasks of buffer P.
  auto col_sum = [&](const char* P, int c) {
    std::string ex;
    for (int t = 0; t < ntask; ++t) ex += (t ? " + " : "") + F("%s[(i64)%d * eps + el_]", P, t * V + c);
    return ex;
  };
  for (int q = 0; q < K; ++q) o.line(F("real gp%d = R(0);", q));
  for (const char* P : {"epa", "epb", "epc"}) {
    o.open(F("if (%s)", P));
    for (int q = 0; q < K; ++q) o.line(F("gp%d += ", q) + col_sum(P, q) + ";");
    o.close();
  }
  o.open("if (gphi)");
  for (int q = 0; q < K; ++q) o.line(F("gphi[(i64)e * %d + %d] = gp%d;", K, q, q));
  o.close();
  // pb1 (nullable): the first-order phi-bar, the phi-bar columns of the first-order pass.
  o.open("if (pb1 && epw)");
  for (int q = 0; q < K; ++q) o.line(F("pb1[(i64)e * %d + %d] = ", K, q) + col_sum("epw", q) + ";");
  o.close();
  o.line("if (!gev) return;");
  emit_ebar_dot(o, p, [&] {
    for (int m = 0; m < Yd; ++m) o.line(F("ybd[%d] = R(0); ybw[%d] = R(0);", m, m));
    for (const char* P : {"epa", "epb", "epc"}) {
      o.open(F("if (%s)", P));
      for (int m = 0; m < Yd; ++m) o.line(F("ybd[%d] += ", m) + col_sum(P, K + m) + ";");
      o.close();
    }
    o.open("if (epw)");
    for (int m = 0; m < Yd; ++m) o.line(F("ybw[%d] = ", m) + col_sum("epw", K + m) + ";");
    o.close();
  });
  o.line("gev[3 * (i64)e] = gx; gev[3 * (i64)e + 1] = gy; gev[3 * (i64)e + 2] = gz;");
  o.close();
}

}  // namespace gen

// Family "uvw_rdbl" of a fully connected plan with an in-kernel radial basis:
//   cgtp_radial_vals (lane = edge): phi(|r|) and phidot = phi'(|r|) (r-hat . rdot) of every edge of
//     [e0, e1) into E x K arrays (the inputs of the double backward run on the plan without a basis);
//   cgtp_radial_dedge (lane = edge): adds to e-bar-dot the chain through phi, J_phi^T phi-bar-dot =
//     (sum gphi_q phi'_q) r-hat, and the curvature grad_r [s (r-hat . rdot)] = s' t r-hat +
//     s (rdot - t r-hat) / |r| with s = sum pb_q phi'_q, s' = sum pb_q phi''_q, t = r-hat . rdot,
//     pb the first-order phi-bar.
std::string generate_uvw_radial_dbl_source(const Plan& p, std::string* err) {
  if (p.mode != CGTP_FULLY_CONNECTED || !p.radial) {
    *err = "family uvw_rdbl is generated for fully connected plans with a radial basis";
    return "";
  }
  const int K = p.K;
  Out o;
  prelude(o, p, false, true);
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_radial_vals(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ vev, const real* __restrict__ vpos, int e0,"
         " int e1, real* __restrict__ phi, real* __restrict__ vphi)");
  o.line("const int e = e0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  emit_edge_vector(o);
  emit_edge_direction(o);
  o.line("const real rr = sqrt(rx * rx + ry * ry + rz * rz), inv = R(1) / rr;");
  o.line("const real nv = (rx * vex + ry * vey + rz * vez) * inv;");
  o.line(F("real fr[%d], dfr[%d];", K, K));
  o.line("radial_eval(rr, fr, dfr, nullptr);");
  for (int q = 0; q < K; ++q) {
    o.line(F("phi[(i64)e * %d + %d] = fr[%d];", K, q, q));
    o.line(F("vphi[(i64)e * %d + %d] = dfr[%d] * nv;", K, q, q));
  }
  o.close();
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_radial_dedge(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ vev, const real* __restrict__ vpos,"
         " const real* __restrict__ gphi, const real* __restrict__ pb, int e0, int e1, real* __restrict__ gev)");
  o.line("const int e = e0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  emit_edge_vector(o);
  emit_edge_direction(o);
  o.line("const real rr = sqrt(rx * rx + ry * ry + rz * rz), inv = R(1) / rr;");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line("const real nv = nx * vex + ny * vey + nz * vez;");
  o.line(F("real fr[%d], dfr[%d], d2fr[%d];", K, K, K));
  o.line("radial_eval(rr, fr, dfr, d2fr);");
  o.line("real sc = R(0), s1 = R(0), s2 = R(0);");
  for (int q = 0; q < K; ++q) {
    o.line(F("sc = fma(gphi[(i64)e * %d + %d], dfr[%d], sc);", K, q, q));
    o.line(F("s1 = fma(pb[(i64)e * %d + %d], dfr[%d], s1);", K, q, q));
    o.line(F("s2 = fma(pb[(i64)e * %d + %d], d2fr[%d], s2);", K, q, q));
  }
  o.line("const real cn = sc + (s2 - s1 * inv) * nv, cv = s1 * inv;");
  o.line("gev[3 * (i64)e] += cn * nx + cv * vex;");
  o.line("gev[3 * (i64)e + 1] += cn * ny + cv * vey;");
  o.line("gev[3 * (i64)e + 2] += cn * nz + cv * vez;");
  o.close();
  emit_small_kernels(o);
  return o.s.str();
}

}  // namespace cgtp
