// Source generator for the gfx950 kernels of one plan.
//
// Everything a plan fixes (paths, block offsets, multiplicities, radial width, the sparse CG
// terms and their coefficients) is emitted as compile-time structure: loops over paths and
// components are unrolled and CG coefficients are literals (LunaTP section 4.3, "sparse
// expansion"; Sobek section 4.5 compiles the same information).  Only the graph stays a
// run-time input.
//
// Channelwise data flow (one wave = 64 lanes = 64 channels):
//   prep      (lane = edge):    r = pos[j] - pos[i] + shift, Y(r/|r|), and the channel-
//                               independent folded coefficients G_pi[m1,m3] = sum_m2 c Y[m2] of
//                               every path, one row per edge in a workspace chunk;
//   fwd       (lane = channel): receiver-major (LunaTP section 4.1); per incoming edge, G and
//                               phi arrive through scalar loads (wave-uniform), x_j through
//                               coalesced vector loads, w = phi A_pi with A in registers, and
//                               the output block accumulates in registers; one store per value;
//   bwd_recv  (lane = channel): receiver-major backward (Sobek section 3.2, Eqs. 18-20, 22):
//                               h = <mbar_i, T_pi>, A-bar partials in registers, and per edge
//                               the cross-channel sums phi-bar and Y-bar, reduced across the
//                               wave by lane swaps and DPP and written once per edge and task;
//   bwd_src   (lane = channel): source-major x-bar (Eq. 21) over the source CSR, one fixed
//                               summation order per sender, no atomics;
//   edge_final(lane = edge):    sums the per-task partials of an edge in a fixed order and
//                               applies the spherical-harmonic Jacobian for the edge-vector
//                               gradient;
//   pos_grad  (lane = node):    position gradient from the two CSRs;
//   a_reduce:                   fixed-order sum of the per-wave A-bar partials.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <set>
#include <sstream>

#include "kernels.hpp"
#include "plan.hpp"

namespace cgtp {
namespace {

std::string F(const char* fmt, ...) {
  char buf[2048];
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

// Register budget: A coefficients held per lane for one subset of paths.
constexpr int kRegBudget = 64;

std::vector<std::vector<int>> subsets(const Plan& p, const std::vector<int>& paths) {
  std::vector<std::vector<int>> out;
  for (int pi : paths) {
    if (out.empty() || int(out.back().size() + 1) * p.K > kRegBudget) out.push_back({});
    out.back().push_back(pi);
  }
  return out;
}

void prelude(Out& o, const Plan& p, bool dual, bool reduce) {
  const bool f64 = p.dtype == CGTP_F64;
  o.line(f64 ? "typedef double real;" : "typedef float real;");
  o.line("typedef long long i64;");
  o.line("#define R(v) ((real)(v))");
  o.line("#define DEV static __device__ __forceinline__");
  if (f64)
    o.line("struct __attribute__((aligned(16))) V4 { real a, b; };  // 16-byte store unit");
  else
    o.line("struct __attribute__((aligned(16))) V4 { real a, b, c, d; };  // 16-byte store unit");
  o.line("extern \"C\" __global__ void __launch_bounds__(256) cgtp_fill_zero(real* __restrict__ p, i64 n) {");
  o.line("  i64 k = (i64)blockIdx.x * 256 + threadIdx.x;");
  o.line("  if (k < n) p[k] = R(0);");
  o.line("}");
  if (dual) {
    // Forward-mode dual numbers with the three partials d/dx, d/dy, d/dz.
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
  if (reduce) {
    // Cross-lane helpers.  swap32(a, b): a <- [a lanes 0-31, b lanes 0-31], b <- [a 32-63, b 32-63];
    // swap16 does the same between odd rows of a and even rows of b; rowsum leaves in every lane the
    // sum of its 16-lane row.
    // The lane swaps go through inline assembly with both registers tied: this compiler's
    // __builtin_amdgcn_permlane{16,32}_swap return the new first operand for both results.
    o.line("DEV void swp32(unsigned& a, unsigned& b) { asm volatile(\"s_nop 1\\n\\tv_permlane32_swap_b32 %0, %1"
           "\\n\\ts_nop 1\" : \"+v\"(a), \"+v\"(b)); }");
    o.line("DEV void swp16(unsigned& a, unsigned& b) { asm volatile(\"s_nop 1\\n\\tv_permlane16_swap_b32 %0, %1"
           "\\n\\ts_nop 1\" : \"+v\"(a), \"+v\"(b)); }");
    if (!f64) {
      for (const char* w : {"32", "16"})
        o.line(F("DEV void swap%s(real& a, real& b) { unsigned x = __builtin_bit_cast(unsigned, a),"
                 " y = __builtin_bit_cast(unsigned, b); swp%s(x, y); a = __builtin_bit_cast(real, x);"
                 " b = __builtin_bit_cast(real, y); }", w, w));
      o.line("template <int C> DEV real dpp(real v) { return __builtin_bit_cast(real, "
             "__builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), C, 0xF, 0xF, false)); }");
    } else {
      for (const char* w : {"32", "16"})
        o.line(F("DEV void swap%s(real& a, real& b) { unsigned long long x = __builtin_bit_cast(unsigned long long, a),"
                 " y = __builtin_bit_cast(unsigned long long, b); unsigned xl = (unsigned)x, xh = (unsigned)(x >> 32),"
                 " yl = (unsigned)y, yh = (unsigned)(y >> 32); swp%s(xl, yl); swp%s(xh, yh);"
                 " a = __builtin_bit_cast(real, (unsigned long long)xl | ((unsigned long long)xh << 32));"
                 " b = __builtin_bit_cast(real, (unsigned long long)yl | ((unsigned long long)yh << 32)); }", w, w, w));
      o.line("template <int C> DEV real dpp(real v) { unsigned long long x = __builtin_bit_cast(unsigned long long, v);");
      o.line("  unsigned lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)x, C, 0xF, 0xF, false);");
      o.line("  unsigned hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(x >> 32), C, 0xF, 0xF, false);");
      o.line("  return __builtin_bit_cast(real, (unsigned long long)lo | ((unsigned long long)hi << 32)); }");
    }
    o.line("DEV real rowsum(real v) { v += dpp<0xB1>(v); v += dpp<0x4E>(v); v += dpp<0x141>(v);"
           " v += dpp<0x140>(v); return v; }");
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

// Edge vector r = pos[send] - pos[recv] (+ shift) of sorted edge e, into rx, ry, rz.
void emit_edge_vector(Out& o) {
  o.line("const int ri = recv[e], sj = send[e];");
  o.line("real rx = pos[3 * (i64)sj] - pos[3 * (i64)ri];");
  o.line("real ry = pos[3 * (i64)sj + 1] - pos[3 * (i64)ri + 1];");
  o.line("real rz = pos[3 * (i64)sj + 2] - pos[3 * (i64)ri + 2];");
  o.open("if (shift)");
  o.line("rx += shift[3 * (i64)e]; ry += shift[3 * (i64)e + 1]; rz += shift[3 * (i64)e + 2];");
  o.close();
}

// prep: lane = edge; writes the G row of every edge of [e0, e1) at G + (e - e0) * stride.
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
  o.line(F("V4* __restrict__ dst = (V4*)(G + (i64)(e - e0) * %d);", p.g_stride));
  const int per = p.dtype == CGTP_F64 ? 2 : 4;
  std::vector<std::string> vals;
  for (const Path& P : p.paths) {
    int s = P.l2 * P.l2;
    for (const GPair& gp : P.gpairs) {
      std::string ex;
      for (auto& t : gp.terms) {
        if (!ex.empty()) ex += " + ";
        ex += lit(t.second) + " * Y[" + std::to_string(s + t.first) + "]";
      }
      vals.push_back(ex);
    }
  }
  while (int(vals.size()) < p.g_stride) vals.push_back("R(0)");
  for (int k = 0; k < p.g_stride; k += per) {
    std::string v;
    for (int t = 0; t < per; ++t) v += (t ? ", " : "") + vals[k + t];
    o.line(F("dst[%d] = V4{", k / per) + v + "};");
  }
  o.close();
}

int path_cost(const Plan& p, const Path& P) {
  return p.K + int(P.gpairs.size()) + std::min(2 * P.l1 + 1, 2 * P.l3 + 1);
}

int out_group_cost(const Plan& p, int k) {
  int c = 0;
  for (int pi : p.by_out[k]) c += path_cost(p, p.paths[pi]);
  return c;
}

std::vector<int> in_blocks_of(const Plan& p, const std::vector<int>& paths) {
  std::set<int> s;
  for (int pi : paths) s.insert(p.paths[pi].i_in);
  return std::vector<int>(s.begin(), s.end());
}

std::vector<int> out_blocks_of(const Plan& p, const std::vector<int>& paths) {
  std::set<int> s;
  for (int pi : paths) s.insert(p.paths[pi].i_out);
  return std::vector<int>(s.begin(), s.end());
}

// x_j components of the input blocks used by `paths`, named x<block>_<m>.
void emit_x_loads(Out& o, const Plan& p, const std::vector<int>& paths) {
  for (int b : in_blocks_of(p, paths)) {
    const Block& B = p.in[b];
    for (int m = 0; m < B.dim(); ++m) o.line(F("const real x%d_%d = xj[%d];", b, m, B.offset + m * B.mul));
  }
}

void emit_a_loads(Out& o, const Plan& p, const std::vector<int>& paths) {
  for (int pi : paths) {
    const Path& P = p.paths[pi];
    for (int q = 0; q < p.K; ++q) o.line(F("const real a%d_%d = A[%d + uc];", pi, q, q * p.n_w + P.w_off));
  }
}

void emit_w(Out& o, const Plan& p, int pi) {
  o.line(F("real w%d = f0 * a%d_0;", pi, pi));
  for (int q = 1; q < p.K; ++q) o.line(F("w%d = fma(f%d, a%d_%d, w%d);", pi, q, pi, q, pi));
}

// acc<m3> += w * sum_m1 G[m1,m3] x[m1] for path pi, choosing where to apply w by cost.
void emit_path_accumulate(Out& o, const Plan& p, int pi) {
  const Path& P = p.paths[pi];
  const int d1 = 2 * P.l1 + 1, d3 = 2 * P.l3 + 1;
  if (d1 <= d3) {
    for (int m = 0; m < d1; ++m) o.line(F("const real s%d_%d = w%d * x%d_%d;", pi, m, pi, P.i_in, m));
    for (size_t t = 0; t < P.gpairs.size(); ++t)
      o.line(F("acc%d = fma(g[%d], s%d_%d, acc%d);", P.gpairs[t].m3, P.g_off + int(t), pi, P.gpairs[t].m1,
               P.gpairs[t].m3));
  } else {
    std::vector<bool> started(d3, false);
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
      if (!started[m3])
        o.line(F("real t%d_%d = g[%d] * x%d_%d;", pi, m3, P.g_off + int(t), P.i_in, m1));
      else
        o.line(F("t%d_%d = fma(g[%d], x%d_%d, t%d_%d);", pi, m3, P.g_off + int(t), P.i_in, m1, pi, m3));
      started[m3] = true;
    }
    for (int m = 0; m < d3; ++m)
      if (started[m]) o.line(F("acc%d = fma(w%d, t%d_%d, acc%d);", m, pi, pi, m, m));
  }
}

const char* kFwdArgs =
    "const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
    " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
    " real* __restrict__ out";

// Channelwise conventional forward of task (output block k, channel block cb) for one receiver.
// Paths are processed in register-budgeted subsets, each re-walking the receiver's edges.
void emit_fwd_task(Out& o, const Plan& p, int ti, const Task& T) {
  const Block& OB = p.out[T.group];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  o.open(F("DEV void fwd_t%d(%s, int node, int e_base)", ti, kFwdArgs));
  o.line(F("const int u = %d + (int)threadIdx.x;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d3; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  for (const auto& S : subsets(p, T.paths)) {
    o.open("");
    emit_a_loads(o, p, S);
    o.open("for (int e = e0; e < e1; ++e)");
    o.line("const int j = col[e];");
    o.line(F("const real* __restrict__ ph = phi + (i64)e * %d;", K));
    o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", p.g_stride));
    o.line(F("const real* __restrict__ xj = x + (i64)j * %d + uc;", p.c_in));
    for (int q = 0; q < K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
    emit_x_loads(o, p, S);
    for (int pi : S) {
      emit_w(o, p, pi);
      emit_path_accumulate(o, p, pi);
    }
    o.close();
    o.close();
  }
  o.open(F("if (u < %d)", MUL));
  o.line(F("real* __restrict__ dst = out + (i64)node * %d + %d + u;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("dst[%d] = acc%d;", m * MUL, m));
  o.close();
  o.close();
}

// Channelwise streamed forward (Sobek Eqs. 33-34): per path, the receiver state
// S[q][m3] = sum_j phi_q C_pi[m3] over the incoming edges, then m += sum_q S[q] A[q, pi, u].
void emit_fwd_streamed_task(Out& o, const Plan& p, int ti, const Task& T) {
  const Block& OB = p.out[T.group];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  o.open(F("DEV void fwds_t%d(%s, int node, int e_base)", ti, kFwdArgs));
  o.line(F("const int u = %d + (int)threadIdx.x;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d3; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  for (int pi : T.paths) {
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
      if (!started[m3])
        o.line(F("real c%d = g[%d] * x%d_%d;", m3, P.g_off + int(t), P.i_in, m1));
      else
        o.line(F("c%d = fma(g[%d], x%d_%d, c%d);", m3, P.g_off + int(t), P.i_in, m1, m3));
      started[m3] = true;
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

// One receiver per block.  Blocks are spread over the 8 XCDs round-robin by the hardware; this
// mapping gives each XCD a contiguous receiver range (spatial neighbours, whose senders' rows
// then stay in that XCD's L2) and runs the tasks in decreasing cost order inside it (LunaTP
// section 4.2, task ordering).
void emit_node_dispatch(Out& o, const std::string& kname, const std::string& args, const std::string& call,
                        int ntask) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open(kname + "(" + args + ", int i0, int nrec, int per, int e_base)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, il = s - t * per;");
  o.line("const int i = xcd * per + il;");
  o.line("if (i >= nrec) return;");
  o.line("const int node = i0 + i;");
  o.open("switch (t)");
  for (int k = 0; k < ntask; ++k) o.line(F("case %d: %s%d(%s, node, e_base); break;", k, call.c_str(), k,
                                          "x, phi, A, G, row_ptr, col, out"));
  o.line("default: break;");
  o.close();
  o.close();
}

// ------------------------------------------------------------------------------ backward

const char* kRecvArgs =
    "const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
    " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
    " const real* __restrict__ gout, real* __restrict__ ep, real* __restrict__ ap";

// Receiver-major backward of task (output block k, path subset, channel block) over the
// receivers [n0, n1).  Per edge: h_pi = <mbar, T_pi> (Eq. 18), phi-bar partials sum_pi A h (Eq. 20)
// and Y-bar partials sum_pi w sum c x mbar (Eq. 22), reduced over the 64 channels of the wave
// and stored in slot `ti` of the edge's partial row.  A-bar = sum_e phi h (Eq. 19) accumulates in
// registers over all edges of the range and is added to the wave's partial slot at the end.
void emit_bwd_recv_task(Out& o, const Plan& p, int ti, const Task& T, int V) {
  const Block& OB = p.out[T.group];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  const int ROW = int(recv_backward_tasks(p).size()) * V;
  o.open(F("DEV void bwr_t%d(%s, int n0, int n1, int e_base, int slot)", ti, kRecvArgs));
  o.line("const int lane = (int)threadIdx.x;");
  o.line(F("const int u = %d + lane;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  emit_a_loads(o, p, T.paths);
  for (int pi : T.paths)
    for (int q = 0; q < K; ++q) o.line(F("real aa%d_%d = R(0);", pi, q));
  o.open("for (int node = n0; node < n1; ++node)");
  o.line(F("const real* __restrict__ gr = gout + (i64)node * %d + %d + uc;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("const real mb%d = u < %d ? gr[%d] : R(0);", m, MUL, m * MUL));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  o.open("for (int e = e0; e < e1; ++e)");
  o.line("const int j = col[e];");
  o.line(F("const real* __restrict__ ph = phi + (i64)e * %d;", K));
  o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", p.g_stride));
  o.line(F("const real* __restrict__ xj = x + (i64)j * %d + uc;", p.c_in));
  for (int q = 0; q < K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
  emit_x_loads(o, p, T.paths);
  for (int v = 0; v < V; ++v) o.line(F("real v%d = R(0);", v));
  for (int pi : T.paths) {
    const Path& P = p.paths[pi];
    const int s = K + P.l2 * P.l2;  // Y-bar slot of this path's SH block
    std::vector<bool> started(d3, false);
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
      if (!started[m3])
        o.line(F("real t%d_%d = g[%d] * x%d_%d;", pi, m3, P.g_off + int(t), P.i_in, m1));
      else
        o.line(F("t%d_%d = fma(g[%d], x%d_%d, t%d_%d);", pi, m3, P.g_off + int(t), P.i_in, m1, pi, m3));
      started[m3] = true;
    }
    bool first = true;
    for (int m = 0; m < d3; ++m)
      if (started[m]) {
        if (first) o.line(F("real h%d = mb%d * t%d_%d;", pi, m, pi, m));
        else o.line(F("h%d = fma(mb%d, t%d_%d, h%d);", pi, m, pi, m, pi));
        first = false;
      }
    emit_w(o, p, pi);
    for (int q = 0; q < K; ++q) {
      o.line(F("aa%d_%d = fma(f%d, h%d, aa%d_%d);", pi, q, q, pi, pi, q));
      o.line(F("v%d = fma(a%d_%d, h%d, v%d);", q, pi, q, pi, q));
    }
    std::set<int> m3used;
    for (auto& gp : P.gpairs) m3used.insert(gp.m3);
    for (int m : m3used) o.line(F("const real wm%d_%d = w%d * mb%d;", pi, m, pi, m));
    for (auto& gp : P.gpairs) {
      o.line(F("{ const real z = x%d_%d * wm%d_%d;", P.i_in, gp.m1, pi, gp.m3));
      for (auto& t : gp.terms) o.line(F("  v%d = fma(%s, z, v%d);", s + t.first, lit(t.second).c_str(), s + t.first));
      o.line("}");
    }
  }
  // Transpose-reduce the V partial sums over the 64 lanes.
  const int H = V / 2, Q = V / 4;
  for (int k = 0; k < H; ++k) o.line(F("swap32(v%d, v%d); v%d += v%d;", k, k + H, k, k + H));
  for (int k = 0; k < Q; ++k) o.line(F("swap16(v%d, v%d); v%d += v%d;", k, k + Q, k, k + Q));
  for (int k = 0; k < Q; ++k) o.line(F("v%d = rowsum(v%d);", k, k));
  o.open("if ((lane & 15) == 0)");
  o.line(F("real* __restrict__ dst = ep + (i64)(e - e_base) * %d + %d + (lane >> 4) * %d;", ROW, ti * V, Q));
  for (int k = 0; k < Q; ++k) o.line(F("dst[%d] = v%d;", k, k));
  o.close();
  o.close();  // edges
  o.close();  // nodes
  o.open(F("if (u < %d)", MUL));
  o.line(F("real* __restrict__ dst = ap + (i64)slot * %d + u;", K * p.n_w));
  for (int pi : T.paths)
    for (int q = 0; q < K; ++q)
      o.line(F("dst[%d] += aa%d_%d;", q * p.n_w + p.paths[pi].w_off, pi, q));
  o.close();
  o.close();
}

// Receiver ranges of R nodes per wave: block b -> XCD b & 7, and inside it (task, range).
void emit_recv_dispatch(Out& o, int ntask) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open(std::string("cgtp_bwd_recv(") + kRecvArgs + ", int i0, int nrec, int per, int nch, int rpw, int e_base)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / nch, c = s - t * nch;");
  o.line("const int lo = xcd * per + c * rpw;");
  o.line("int hi = lo + rpw; if (hi > (xcd + 1) * per) hi = (xcd + 1) * per; if (hi > nrec) hi = nrec;");
  o.line("if (lo >= hi) return;");
  o.line("const int slot = xcd * nch + c;");
  o.open("switch (t)");
  for (int k = 0; k < ntask; ++k)
    o.line(F("case %d: bwr_t%d(x, phi, A, G, row_ptr, col, gout, ep, ap, i0 + lo, i0 + hi, e_base, slot); break;",
             k, k));
  o.line("default: break;");
  o.close();
  o.close();
}

const char* kSrcArgs =
    "const real* __restrict__ phi, const real* __restrict__ A, const real* __restrict__ G,"
    " const real* __restrict__ gout, const int* __restrict__ recv, const int* __restrict__ src_ptr,"
    " const int* __restrict__ src_edge, real* __restrict__ gx";

// Source-major x-bar of task (input block b, channel block cb) for one sender (Eq. 21):
// x-bar_j[m1] = sum over out-edges, paths of w_pi sum_m3 G[m1,m3] mbar_i[m3].
void emit_bwd_src_task(Out& o, const Plan& p, int ti, const Task& T) {
  const Block& IB = p.in[T.group];
  const int d1 = IB.dim(), MUL = IB.mul, K = p.K;
  o.open(F("DEV void bws_t%d(%s, int node, int e_base, int accumulate)", ti, kSrcArgs));
  o.line(F("const int u = %d + (int)threadIdx.x;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d1; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int s0 = src_ptr[node], s1 = src_ptr[node + 1];");
  for (const auto& S : subsets(p, T.paths)) {
    o.open("");
    emit_a_loads(o, p, S);
    o.open("for (int k = s0; k < s1; ++k)");
    o.line("const int e = src_edge[k];");
    o.line("const int i = recv[e];");
    o.line(F("const real* __restrict__ ph = phi + (i64)e * %d;", K));
    o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", p.g_stride));
    o.line(F("const real* __restrict__ gi = gout + (i64)i * %d + uc;", p.c_out));
    for (int q = 0; q < K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
    for (int ob : out_blocks_of(p, S)) {
      const Block& B = p.out[ob];
      for (int m = 0; m < B.dim(); ++m) o.line(F("const real mb%d_%d = gi[%d];", ob, m, B.offset + m * B.mul));
    }
    for (int pi : S) {
      const Path& P = p.paths[pi];
      const int d3 = 2 * P.l3 + 1;
      emit_w(o, p, pi);
      if (d3 <= d1) {
        for (int m = 0; m < d3; ++m) o.line(F("const real s%d_%d = w%d * mb%d_%d;", pi, m, pi, P.i_out, m));
        for (size_t t = 0; t < P.gpairs.size(); ++t)
          o.line(F("acc%d = fma(g[%d], s%d_%d, acc%d);", P.gpairs[t].m1, P.g_off + int(t), pi, P.gpairs[t].m3,
                   P.gpairs[t].m1));
      } else {
        std::vector<bool> started(d1, false);
        for (size_t t = 0; t < P.gpairs.size(); ++t) {
          int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
          if (!started[m1])
            o.line(F("real b%d_%d = g[%d] * mb%d_%d;", pi, m1, P.g_off + int(t), P.i_out, m3));
          else
            o.line(F("b%d_%d = fma(g[%d], mb%d_%d, b%d_%d);", pi, m1, P.g_off + int(t), P.i_out, m3, pi, m1));
          started[m1] = true;
        }
        for (int m = 0; m < d1; ++m)
          if (started[m]) o.line(F("acc%d = fma(w%d, b%d_%d, acc%d);", m, pi, pi, m, m));
      }
    }
    o.close();
    o.close();
  }
  o.open(F("if (u < %d)", MUL));
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

void emit_src_dispatch(Out& o, int ntask) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open(std::string("cgtp_bwd_src(") + kSrcArgs + ", int nrec, int per, int e_base, int accumulate)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, il = s - t * per;");
  o.line("const int node = xcd * per + il;");
  o.line("if (node >= nrec) return;");
  o.open("switch (t)");
  for (int k = 0; k < ntask; ++k)
    o.line(F("case %d: bws_t%d(phi, A, G, gout, recv, src_ptr, src_edge, gx, node, e_base, accumulate); break;", k,
             k));
  o.line("default: break;");
  o.close();
  o.close();
}

// Per-edge finalisation: phi-bar and Y-bar = fixed-order sums of the task partials, then the
// edge-vector gradient e-bar = J_Y(r)^T Y-bar with J_Y = (I - n n^T) dY/dn / |r|.
void emit_edge_final(Out& o, const Plan& p, int ntask, int V) {
  const int K = p.K, ROW = ntask * V;
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_edge_final(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ ep, int e0, int e1, real* __restrict__ gphi,"
         " real* __restrict__ gev)");
  o.line("const int e = e0 + (int)(blockIdx.x * 256 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  o.line(F("const real* __restrict__ row = ep + (i64)(e - e0) * %d;", ROW));
  o.open("if (gphi)");
  for (int q = 0; q < K; ++q) {
    std::string ex = F("row[%d]", q);
    for (int t = 1; t < ntask; ++t) ex += F(" + row[%d]", t * V + q);
    o.line(F("gphi[(i64)e * %d + %d] = ", K, q) + ex + ";");
  }
  o.close();
  o.line("if (!gev) return;");
  emit_edge_vector(o);
  o.line("const real inv = R(1) / sqrt(rx * rx + ry * ry + rz * rz);");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line(F("D3 Y[%d];", p.sh_dim));
  o.line("sh_eval<D3>(D3(nx, R(1), R(0), R(0)), D3(ny, R(0), R(1), R(0)), D3(nz, R(0), R(0), R(1)), Y);");
  o.line("real gx = R(0), gy = R(0), gz = R(0);");
  for (int m = 0; m < p.sh_dim; ++m) {
    std::string ex = F("row[%d]", K + m);
    for (int t = 1; t < ntask; ++t) ex += F(" + row[%d]", t * V + K + m);
    o.line(F("{ const real yb = ") + ex + F("; gx = fma(yb, Y[%d].x, gx); gy = fma(yb, Y[%d].y, gy);"
                                             " gz = fma(yb, Y[%d].z, gz); }", m, m, m));
  }
  o.line("const real d = nx * gx + ny * gy + nz * gz;");
  o.line("gev[3 * (i64)e] = (gx - nx * d) * inv;");
  o.line("gev[3 * (i64)e + 1] = (gy - ny * d) * inv;");
  o.line("gev[3 * (i64)e + 2] = (gz - nz * d) * inv;");
  o.close();
}

void emit_small_kernels(Out& o) {
  // pos-bar_i = sum over out-edges of e-bar - sum over in-edges of e-bar (fixed CSR order).
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_pos_grad(const real* __restrict__ gev, const int* __restrict__ row_ptr,"
         " const int* __restrict__ src_ptr, const int* __restrict__ src_edge, int n, real* __restrict__ gpos)");
  o.line("const int i = (int)(blockIdx.x * 256 + threadIdx.x);");
  o.line("if (i >= n) return;");
  o.line("real sx = R(0), sy = R(0), sz = R(0);");
  o.open("for (int k = src_ptr[i]; k < src_ptr[i + 1]; ++k)");
  o.line("const i64 e = src_edge[k];");
  o.line("sx += gev[3 * e]; sy += gev[3 * e + 1]; sz += gev[3 * e + 2];");
  o.close();
  o.open("for (i64 e = row_ptr[i]; e < row_ptr[i + 1]; ++e)");
  o.line("sx -= gev[3 * e]; sy -= gev[3 * e + 1]; sz -= gev[3 * e + 2];");
  o.close();
  o.line("gpos[3 * (i64)i] = sx; gpos[3 * (i64)i + 1] = sy; gpos[3 * (i64)i + 2] = sz;");
  o.close();
  // A-bar = sum over wave slots of the partials, slot order fixed.
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_a_reduce(const real* __restrict__ ap, int nslot, int n, real* __restrict__ gA)");
  o.line("const int k = (int)(blockIdx.x * 256 + threadIdx.x);");
  o.line("if (k >= n) return;");
  o.line("real s = R(0);");
  o.line("for (int w = 0; w < nslot; ++w) s += ap[(i64)w * n + k];");
  o.line("gA[k] = s;");
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
    for (int c = 0; c < ncb; ++c) t.push_back({k, c, p.by_out[k]});
  }
  return t;
}

std::vector<Task> recv_backward_tasks(const Plan& p) {
  std::vector<Task> t;
  for (const Task& f : forward_tasks(p))
    for (const auto& S : subsets(p, f.paths)) t.push_back({f.group, f.cb, S});
  return t;
}

std::vector<Task> source_tasks(const Plan& p) {
  std::vector<Task> t;
  for (int k = 0; k < int(p.in.size()); ++k) {
    if (p.by_in[k].empty()) continue;
    int ncb = (p.in[k].mul + 63) / 64;
    for (int c = 0; c < ncb; ++c) t.push_back({k, c, p.by_in[k]});
  }
  return t;
}

int edge_partial_width(const Plan& p) { return (p.K + p.sh_dim + 3) / 4 * 4; }

std::string generate_source(const Plan& p, const std::string& family, std::string* err) {
  Out o;
  if (p.mode != CGTP_CHANNELWISE) {
    *err = "fully connected kernels are not generated yet";
    return "";
  }
  if (family == "fwd" || family == "fwds") {
    prelude(o, p, false, false);
    emit_sh(o, p.lmax);
    emit_prep(o, p);
    auto tasks = forward_tasks(p);
    bool streamed = family == "fwds";
    for (int k = 0; k < int(tasks.size()); ++k) {
      if (streamed) emit_fwd_streamed_task(o, p, k, tasks[k]);
      else emit_fwd_task(o, p, k, tasks[k]);
    }
    emit_node_dispatch(o, streamed ? "cgtp_fwd_streamed" : "cgtp_fwd", kFwdArgs, streamed ? "fwds_t" : "fwd_t",
                       int(tasks.size()));
    return o.s.str();
  }
  if (family == "bwd") {
    prelude(o, p, true, true);
    emit_sh(o, p.lmax);
    emit_prep(o, p);
    const int V = edge_partial_width(p);
    auto rt = recv_backward_tasks(p);
    for (int k = 0; k < int(rt.size()); ++k) emit_bwd_recv_task(o, p, k, rt[k], V);
    emit_recv_dispatch(o, int(rt.size()));
    auto st = source_tasks(p);
    for (int k = 0; k < int(st.size()); ++k) emit_bwd_src_task(o, p, k, st[k]);
    emit_src_dispatch(o, int(st.size()));
    emit_edge_final(o, p, int(rt.size()), V);
    emit_small_kernels(o);
    return o.s.str();
  }
  *err = "unknown kernel family " + family;
  return "";
}

}  // namespace cgtp
