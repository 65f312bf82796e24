// Source generator for the gfx950 kernels of one plan.
//
// Everything a plan fixes (paths, block offsets, multiplicities, radial width, the sparse CG
// terms and their coefficients) is emitted as compile-time structure: loops over paths and
// components are unrolled, CG coefficients are literals (LunaTP section 4.3, "sparse
// expansion"; Sobek section 4.5 compiles the same information).  Only the graph stays a
// run-time input.
//
// Data flow of the channelwise forward (one wave = 64 lanes = 64 channels of one receiver
// and one output block, LunaTP section 4.1 node-centric execution with Sobek's output group):
//   prep  (lane = edge):   r = pos[j] - pos[i] + shift, Y(r/|r|), and the channel-independent
//                           folded coefficients G_pi[m1,m3] = sum_m2 c[m1,m2,m3] Y[m2] of every
//                           path, one row per edge in a chunk of the workspace;
//   fwd   (lane = channel): for each incoming edge (receiver CSR order), G and phi are read
//                           with scalar loads (wave-uniform), x_j with coalesced vector loads,
//                           w = phi A_pi (A in registers), and the output components accumulate
//                           in registers; one store per output value, no atomics.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <sstream>

#include "kernels.hpp"
#include "plan.hpp"

namespace cgtp {
namespace {

std::string F(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return buf;
}

std::string lit(double v) { return F("R(%.17g)", v); }

struct Out {
  std::ostringstream s;
  int ind = 0;
  void line(const std::string& t) {
    for (int k = 0; k < ind; ++k) s << "  ";
    s << t << "\n";
  }
  void open(const std::string& t) {
    line(t + " {");
    ++ind;
  }
  void close(const std::string& t = "}") {
    --ind;
    line(t);
  }
};

long double dfact(int n) {  // n!!
  long double r = 1;
  for (int k = n; k > 1; k -= 2) r *= k;
  return r;
}
long double fct(int n) {
  long double r = 1;
  for (int k = 2; k <= n; ++k) r *= k;
  return r;
}

void prelude(Out& o, const Plan& p, bool dual) {
  o.line(p.dtype == CGTP_F64 ? "typedef double real;" : "typedef float real;");
  o.line("typedef long long i64;");
  o.line("#define R(v) ((real)(v))");
  o.line("#define DEV static __device__ __forceinline__");
  if (p.dtype == CGTP_F64)
    o.line("struct __attribute__((aligned(16))) V4 { real a, b; };  // 16-byte store unit");
  else
    o.line("struct __attribute__((aligned(16))) V4 { real a, b, c, d; };  // 16-byte store unit");
  if (dual) {
    // Forward-mode dual numbers with the three partials d/dx, d/dy, d/dz of a unit vector.
    o.line("struct D3 { real v, x, y, z;");
    o.line("  __device__ D3() {}");
    o.line("  __device__ D3(real c) : v(c), x(0), y(0), z(0) {}");
    o.line("  __device__ D3(real a, real b, real c, real d) : v(a), x(b), y(c), z(d) {} };");
    o.line("DEV D3 operator+(D3 a, D3 b) { return D3(a.v + b.v, a.x + b.x, a.y + b.y, a.z + b.z); }");
    o.line("DEV D3 operator-(D3 a, D3 b) { return D3(a.v - b.v, a.x - b.x, a.y - b.y, a.z - b.z); }");
    o.line("DEV D3 operator*(D3 a, D3 b) { return D3(a.v * b.v, a.x * b.v + a.v * b.x, a.y * b.v + a.v * b.y,"
           " a.z * b.v + a.v * b.z); }");
    o.line("DEV D3 operator*(real c, D3 b) { return D3(c * b.v, c * b.x, c * b.y, c * b.z); }");
  }
}

// Real spherical harmonics up to degree L, component normalised, as the three-term Legendre
// recurrence in z times (x + iy)^m split into real and imaginary parts.  S is real or D3.
void emit_sh(Out& o, int L) {
  o.line("template <typename S>");
  o.open("DEV void sh_eval(S x, S y, S z, S* Y)");
  o.line("S a0 = S(R(1)), b0 = S(R(0));");
  for (int m = 1; m <= L; ++m)
    o.line(F("S a%d = x * a%d - y * b%d, b%d = x * b%d + y * a%d;", m, m - 1, m - 1, m, m - 1, m - 1));
  for (int m = 0; m <= L; ++m) {
    o.line(F("S q%d_%d = S(%s);", m, m, lit(double(dfact(2 * m - 1))).c_str()));
    if (m + 1 <= L) o.line(F("S q%d_%d = %s * (z * q%d_%d);", m + 1, m, lit(2.0 * m + 1).c_str(), m, m));
    for (int l = m + 2; l <= L; ++l)
      o.line(F("S q%d_%d = %s * (z * q%d_%d) - %s * q%d_%d;", l, m, lit(double(2 * l - 1) / (l - m)).c_str(),
               l - 1, m, lit(double(l + m - 1) / (l - m)).c_str(), l - 2, m));
  }
  for (int l = 0; l <= L; ++l)
    for (int m = 0; m <= l; ++m) {
      long double nrm = std::sqrt((2.0L * l + 1) * fct(l - m) / fct(l + m));
      if (m == 0) {
        o.line(F("Y[%d] = %s * q%d_0;", l * l + l, lit(double(nrm)).c_str(), l));
      } else {
        double c = double(nrm * std::sqrt(2.0L));
        o.line(F("Y[%d] = %s * (q%d_%d * a%d);", l * l + l + m, lit(c).c_str(), l, m, m));
        o.line(F("Y[%d] = %s * (q%d_%d * b%d);", l * l + l - m, lit(c).c_str(), l, m, m));
      }
    }
  o.close();
}

// Edge vector r = pos[send] - pos[recv] (+ shift) of edge e, into rx, ry, rz.
void emit_edge_vector(Out& o) {
  o.line("const int ri = recv[e], sj = send[e];");
  o.line("real rx = pos[3 * (i64)sj] - pos[3 * (i64)ri];");
  o.line("real ry = pos[3 * (i64)sj + 1] - pos[3 * (i64)ri + 1];");
  o.line("real rz = pos[3 * (i64)sj + 2] - pos[3 * (i64)ri + 2];");
  o.open("if (shift)");
  o.line("rx += shift[3 * (i64)e]; ry += shift[3 * (i64)e + 1]; rz += shift[3 * (i64)e + 2];");
  o.close();
}

// prep kernel: lane = edge; writes the G row of every edge of [e0, e1) at G + (e - e0) * stride.
void emit_prep(Out& o, const Plan& p) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_prep(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, int e0, int e1, real* __restrict__ G)");
  o.line("const int e = e0 + (int)(blockIdx.x * 256 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  emit_edge_vector(o);
  o.line("const real inv = R(1) / sqrt(rx * rx + ry * ry + rz * rz);");
  o.line(F("real Y[%d];", p.sh_dim));
  o.line("sh_eval<real>(rx * inv, ry * inv, rz * inv, Y);");
  o.line(F("real g[%d];", p.g_stride));
  for (const Path& P : p.paths) {
    int s = P.l2 * P.l2;
    for (size_t k = 0; k < P.gpairs.size(); ++k) {
      std::string ex;
      for (auto& t : P.gpairs[k].terms) {
        if (!ex.empty()) ex += " + ";
        ex += lit(t.second) + " * Y[" + std::to_string(s + t.first) + "]";
      }
      o.line(F("g[%d] = %s;", P.g_off + int(k), ex.c_str()));
    }
  }
  for (int k = p.g_width; k < p.g_stride; ++k) o.line(F("g[%d] = R(0);", k));
  o.line(F("V4* dst = (V4*)(G + (i64)(e - e0) * %d);", p.g_stride));
  int per = p.dtype == CGTP_F64 ? 2 : 4;
  for (int k = 0; k < p.g_stride; k += per) {
    if (per == 4)
      o.line(F("dst[%d] = V4{g[%d], g[%d], g[%d], g[%d]};", k / 4, k, k + 1, k + 2, k + 3));
    else
      o.line(F("dst[%d] = V4{g[%d], g[%d]};", k / 2, k, k + 1));
  }
  o.close();
}

int out_group_cost(const Plan& p, int k) {
  int c = 0;
  for (int pi : p.by_out[k]) {
    const Path& P = p.paths[pi];
    c += p.K + int(P.gpairs.size()) + std::min(2 * P.l1 + 1, 2 * P.l3 + 1);
  }
  return c;
}

// Per-channel register view of the x blocks of sender j used by a set of paths.
void emit_x_loads(Out& o, const Plan& p, const std::vector<int>& paths) {
  std::vector<int> blocks;
  for (int pi : paths) blocks.push_back(p.paths[pi].i_in);
  std::sort(blocks.begin(), blocks.end());
  blocks.erase(std::unique(blocks.begin(), blocks.end()), blocks.end());
  for (int b : blocks) {
    const Block& B = p.in[b];
    for (int m = 0; m < B.dim(); ++m)
      o.line(F("const real x%d_%d = xj[%d];", b, m, B.offset + m * B.mul));
  }
}

// Channelwise conventional forward of output block k for one receiver and channel block.
void emit_fwd_group(Out& o, const Plan& p, int k) {
  const Block& OB = p.out[k];
  const auto& paths = p.by_out[k];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  o.open(F("DEV void fwd_out%d(const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
           " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
           " real* __restrict__ out, int node, int cb, int e_base)", k));
  o.line("const int u = cb * 64 + (int)threadIdx.x;");
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int pi : paths) {
    const Path& P = p.paths[pi];
    for (int q = 0; q < K; ++q)
      o.line(F("const real a%d_%d = A[%d + uc];", pi, q, q * p.n_w + P.w_off));
  }
  for (int m = 0; m < d3; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  o.open("for (int e = e0; e < e1; ++e)");
  o.line("const int j = col[e];");
  o.line(F("const real* __restrict__ ph = phi + (i64)e * %d;", K));
  o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", p.g_stride));
  o.line(F("const real* __restrict__ xj = x + (i64)j * %d + uc;", p.c_in));
  for (int q = 0; q < K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
  emit_x_loads(o, p, paths);
  for (int pi : paths) {
    const Path& P = p.paths[pi];
    const int d1 = 2 * P.l1 + 1;
    std::string w;
    o.line(F("real w%d = f0 * a%d_0;", pi, pi));
    for (int q = 1; q < K; ++q) o.line(F("w%d = fma(f%d, a%d_%d, w%d);", pi, q, pi, q, pi));
    if (d1 <= d3) {
      for (int m = 0; m < d1; ++m) o.line(F("const real s%d_%d = w%d * x%d_%d;", pi, m, pi, P.i_in, m));
      for (size_t t = 0; t < P.gpairs.size(); ++t)
        o.line(F("acc%d = fma(g[%d], s%d_%d, acc%d);", P.gpairs[t].m3, P.g_off + int(t), pi, P.gpairs[t].m1,
                 P.gpairs[t].m3));
    } else {
      std::vector<bool> started(d3, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (!started[m3]) {
          o.line(F("real t%d_%d = g[%d] * x%d_%d;", pi, m3, P.g_off + int(t), P.i_in, m1));
          started[m3] = true;
        } else {
          o.line(F("t%d_%d = fma(g[%d], x%d_%d, t%d_%d);", pi, m3, P.g_off + int(t), P.i_in, m1, pi, m3));
        }
      }
      for (int m = 0; m < d3; ++m)
        if (started[m]) o.line(F("acc%d = fma(w%d, t%d_%d, acc%d);", m, pi, pi, m, m));
    }
  }
  o.close();
  o.open(F("if (u < %d)", MUL));
  o.line(F("real* __restrict__ dst = out + (i64)node * %d + %d + u;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("dst[%d] = acc%d;", m * MUL, m));
  o.close();
  o.close();
}

// Channelwise streamed forward of output block k (Sobek Eqs. 33-34): for each path of the
// block, accumulate the receiver state S[q][m3] = sum_j phi_q C_pi[m3] over the incoming edges,
// then apply m += sum_q S[q] A[q, pi, u].
void emit_fwd_streamed_group(Out& o, const Plan& p, int k) {
  const Block& OB = p.out[k];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  o.open(F("DEV void fwds_out%d(const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
           " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
           " real* __restrict__ out, int node, int cb, int e_base)", k));
  o.line("const int u = cb * 64 + (int)threadIdx.x;");
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d3; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  for (int pi : p.by_out[k]) {
    const Path& P = p.paths[pi];
    o.open("");
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d3; ++m) o.line(F("real S%d_%d = R(0);", q, m));
    o.open("for (int e = e0; e < e1; ++e)");
    o.line("const int j = col[e];");
    o.line(F("const real* __restrict__ ph = phi + (i64)e * %d;", K));
    o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", p.g_stride));
    o.line(F("const real* __restrict__ xj = x + (i64)j * %d + uc;", p.c_in));
    emit_x_loads(o, p, {pi});
    std::vector<bool> started(d3, false);
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
      if (!started[m3]) {
        o.line(F("real c%d = g[%d] * x%d_%d;", m3, P.g_off + int(t), P.i_in, m1));
        started[m3] = true;
      } else {
        o.line(F("c%d = fma(g[%d], x%d_%d, c%d);", m3, P.g_off + int(t), P.i_in, m1, m3));
      }
    }
    for (int q = 0; q < K; ++q) {
      o.line(F("const real f%d = ph[%d];", q, q));
      for (int m = 0; m < d3; ++m)
        if (started[m]) o.line(F("S%d_%d = fma(f%d, c%d, S%d_%d);", q, m, q, m, q, m));
    }
    o.close();
    for (int q = 0; q < K; ++q) {
      o.line(F("const real a%d = A[%d + uc];", q, q * p.n_w + P.w_off));
      for (int m = 0; m < d3; ++m) o.line(F("acc%d = fma(S%d_%d, a%d, acc%d);", m, q, m, q, m));
    }
    o.close();
  }
  o.open(F("if (u < %d)", MUL));
  o.line(F("real* __restrict__ dst = out + (i64)node * %d + %d + u;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("dst[%d] = acc%d;", m * MUL, m));
  o.close();
  o.close();
}

// Dispatch kernel over tasks (group, channel block) x receivers.  Blocks are spread over the
// 8 XCDs round-robin by the hardware; this mapping gives each XCD a contiguous receiver range
// (spatial neighbours, so their senders' x rows stay in that XCD's L2) and, inside it, runs
// the tasks in decreasing cost order (LunaTP section 4.2, task ordering).
void emit_dispatch(Out& o, const Plan& p, const std::string& kname, const std::string& fprefix,
                   const std::vector<Task>& tasks) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open(kname + "(const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
                 " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
                 " real* __restrict__ out, int i0, int nrec, int per, int e_base)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, il = s - t * per;");
  o.line("const int i = xcd * per + il;");
  o.line("if (i >= nrec) return;");
  o.line("const int node = i0 + i;");
  o.open("switch (t)");
  for (size_t k = 0; k < tasks.size(); ++k)
    o.line(F("case %d: %s%d(x, phi, A, G, row_ptr, col, out, node, %d, e_base); break;", int(k), fprefix.c_str(),
             tasks[k].group, tasks[k].cb));
  o.line("default: break;");
  o.close();
  o.close();
}

}  // namespace

std::vector<Task> forward_tasks(const Plan& p) {
  std::vector<int> order(p.out.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return out_group_cost(p, a) > out_group_cost(p, b); });
  std::vector<Task> t;
  for (int k : order) {
    if (p.by_out[k].empty()) continue;
    int ncb = (p.out[k].mul + 63) / 64;
    for (int c = 0; c < ncb; ++c) t.push_back({k, c});
  }
  return t;
}

std::vector<Task> source_tasks(const Plan& p) {
  std::vector<Task> t;
  for (int k = 0; k < int(p.in.size()); ++k) {
    if (p.by_in[k].empty()) continue;
    int ncb = (p.in[k].mul + 63) / 64;
    for (int c = 0; c < ncb; ++c) t.push_back({k, c});
  }
  return t;
}

std::string generate_source(const Plan& p, const std::string& family, std::string* err) {
  Out o;
  if (family == "fwd" || family == "fwds") {
    if (p.mode != CGTP_CHANNELWISE) {
      *err = "fully connected forward is generated by the uvw family";
      return "";
    }
    prelude(o, p, false);
    emit_sh(o, p.lmax);
    emit_prep(o, p);
    auto tasks = forward_tasks(p);
    bool streamed = family == "fwds";
    for (int k = 0; k < int(p.out.size()); ++k)
      if (!p.by_out[k].empty()) {
        if (streamed)
          emit_fwd_streamed_group(o, p, k);
        else
          emit_fwd_group(o, p, k);
      }
    emit_dispatch(o, p, streamed ? "cgtp_fwd_streamed" : "cgtp_fwd", streamed ? "fwds_out" : "fwd_out", tasks);
    return o.s.str();
  }
  *err = "unknown kernel family " + family;
  return "";
}

}  // namespace cgtp
