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

#include <cstdio>
#include <functional>
#include <map>
#include <memory>
#include <numeric>
#include <set>
#include <sstream>

#include "codegen.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace cgtp {
namespace gen {

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


// Split a task's paths into consecutive subsets whose A coefficients (K per path) fit `avail`
// registers; each subset re-walks the edge list (only tasks of one oversized block need more
// than one).
std::vector<std::vector<int>> a_subsets(const Plan& p, const std::vector<int>& paths, int avail) {
  std::vector<std::vector<int>> out;
  const int per = std::max(1, avail / std::max(1, p.K * (p.dtype == CGTP_F64 ? 2 : 1)));
  for (int pi : paths) {
    if (out.empty() || int(out.back().size()) >= per) out.push_back({});
    out.back().push_back(pi);
  }
  return out;
}

std::vector<std::vector<int>> subsets(const Plan& p, const std::vector<int>& paths) {
  std::vector<std::vector<int>> out;
  for (int pi : paths) {
    if (out.empty() || int(out.back().size() + 1) * p.K > kRegBudget) out.push_back({});
    out.back().push_back(pi);
  }
  return out;
}

void emit_vz(Out& o, const Plan& p) {
  if (p.vec_g) o.line("int vz; asm(\"v_mov_b32 %0, 0\" : \"=v\"(vz));");
}

GStream::GStream(Out& o, const Plan& p, int pi, const std::string& row, const std::string& tag, bool stream)
    : o_(o), p_(p), pi_(pi), row_(row), tag_(tag) {
  const Path& P = p.paths[pi];
  vec_ = path_vec(P);
  per_ = p.dtype == CGTP_F64 ? 2 : 4;
  n_ = (int(P.gpairs.size()) + per_ - 1) / per_;
  if (!vec_) return;
  o.line(F("const V4* __restrict__ gv%s%d = (const V4*)(%s + %d) + vz;", tag.c_str(), pi, row.c_str(), P.g_off));
  if (!stream)
    while (next_ * kGvecChunk < n_) load(next_, false);
}

void GStream::load(int chunk, bool barrier) {
  if (barrier && chunk >= 2) o_.line("__builtin_amdgcn_sched_barrier(0);");
  for (int c = chunk * kGvecChunk; c < std::min(n_, (chunk + 1) * kGvecChunk); ++c)
    o_.line(F("const V4 gq%s%d_%d = gv%s%d[%d];", tag_.c_str(), pi_, c, tag_.c_str(), pi_, c));
  next_ = chunk + 1;
}

std::string GStream::ref(int t) {
  if (!vec_) return gref(p_, pi_, t, row_, tag_, false);
  const int chunk = t / per_ / kGvecChunk;
  while (next_ <= chunk + 1 && next_ * kGvecChunk < n_) load(next_, true);
  return gref(p_, pi_, t, row_, tag_, true);
}

std::string gref(const Plan& p, int pi, int t, const std::string& row, const std::string& tag, bool vec) {
  const Path& P = p.paths[pi];
  if (!vec || !path_vec(P)) return F("%s[%d]", row.c_str(), P.g_off + t);
  const int per = p.dtype == CGTP_F64 ? 2 : 4;
  return F("gq%s%d_%d.%c", tag.c_str(), pi, t / per, "abcd"[t % per]);
}

// Radial basis of |r| (plan.radial 1: Bessel with the p = 6 polynomial envelope, zero beyond the
// cutoff; 2: Gaussians centred at k r_c / (K - 1) with width r_c / (K - 1)), with d/dr when df is
// non-null and d^2/dr^2 (the double backward's curvature term) when d2f is non-null.
void emit_radial(Out& o, const Plan& p) {
  const int K = p.K;
  o.open("DEV void radial_eval(real r, real* f, real* df, real* d2f)");
  if (p.radial == 1) {
    o.line(F("const real rc = R(%.17g), d = r / rc;", p.r_cut));
    o.line("const real d2 = d * d, d4 = d2 * d2, d5 = d4 * d, d6 = d5 * d, d7 = d6 * d, d8 = d7 * d;");
    o.line("const bool in = d < R(1);");
    o.line("const real u = in ? R(1) - R(28) * d6 + R(48) * d7 - R(21) * d8 : R(0);");
    o.line("const real du = in ? (R(-168) * d5 + R(336) * d6 - R(168) * d7) / rc : R(0);");
    o.line("const real d2u = in ? (R(-840) * d4 + R(2016) * d5 - R(1176) * d6) / (rc * rc) : R(0);");
    o.line(F("const real nrm = R(%.17g), ir = R(1) / r;", std::sqrt(2.0 / p.r_cut)));
    o.open(F("for (int n = 0; n < %d; ++n)", K));
    o.line(F("const real a = R(n + 1) * R(%.17g);", M_PI / p.r_cut));
    o.line("const real sn = sin(a * r), cs = cos(a * r);");
    o.line("const real b = nrm * sn * ir, db = nrm * (a * cs * r - sn) * ir * ir;");
    o.line("f[n] = b * u;");
    o.line("if (df) df[n] = db * u + b * du;");
    o.line("if (d2f) d2f[n] = nrm * (R(2) * sn - R(2) * a * r * cs - a * a * r * r * sn) * ir * ir * ir * u"
           " + R(2) * db * du + b * d2u;");
    o.close();
  } else {
    o.line(F("const real D = R(%.17g), inv2 = R(1) / (R(2) * D * D);", p.r_cut / (K - 1)));
    o.open(F("for (int k = 0; k < %d; ++k)", K));
    o.line("const real t = r - R(k) * D, g = exp(-t * t * inv2);");
    o.line("f[k] = g;");
    o.line("if (df) df[k] = -t * R(2) * inv2 * g;");
    o.line("if (d2f) d2f[k] = (R(4) * t * t * inv2 * inv2 - R(2) * inv2) * g;");
    o.close();
  }
  o.close();
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
  if (!f64) {
    // acc += c[lane r of the row] * x and d = c[lane r of the row] * x: the coefficient operand
    // read from lane r of each 16-lane row (DPP row_newbcast), so that each row of a wave can take
    // the coefficients of its own edge from one register.  The register read this way always
    // comes from a memory load, never from a VALU result just before it.
    o.line("#define BFMA(acc, c, x, r) asm(\"v_fmac_f32_dpp %0, %1, %2 row_newbcast:\" #r \" row_mask:0xf bank_mask:0xf\""
           " : \"+v\"(acc) : \"v\"(c), \"v\"(x))");
    o.line("#define BMUL(d, c, x, r) asm(\"v_mul_f32_dpp %0, %1, %2 row_newbcast:\" #r \" row_mask:0xf bank_mask:0xf\""
           " : \"=v\"(d) : \"v\"(c), \"v\"(x))");
    // 64 consecutive coefficients of a row from `base` on, four per lane of each 16-lane row
    // (lane r holds base + 4r .. 4r + 3); lanes past the row's end `lim` (a multiple of 4) read
    // its last four values instead, which no coefficient reference uses.
    o.line("DEV V4 gchunk(const real* __restrict__ g, int base, int lim, int r16) {");
    o.line("  return *(const V4*)(g + min(base + 4 * r16, lim - 4));");
    o.line("}");
  }
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
    // Cross-lane helpers: rowsum leaves in every lane the sum of its 16-lane row (DPP), __shfl_rd
    // reads one lane.  Lane swaps are emitted inline by emit_swaps.
    if (!f64) {
      o.line("template <int C> DEV real dpp(real v) { return __builtin_bit_cast(real, "
             "__builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), C, 0xF, 0xF, false)); }");
    } else {
      o.line("template <int C> DEV real dpp(real v) { unsigned long long x = __builtin_bit_cast(unsigned long long, v);");
      o.line("  unsigned lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)x, C, 0xF, 0xF, false);");
      o.line("  unsigned hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(x >> 32), C, 0xF, 0xF, false);");
      o.line("  return __builtin_bit_cast(real, (unsigned long long)lo | ((unsigned long long)hi << 32)); }");
    }
    if (!f64)
      o.line("DEV real __shfl_rd(real v, int l) { return __builtin_bit_cast(real, "
             "__builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); }");
    else
      o.line("DEV real __shfl_rd(real v, int l) { unsigned long long x = __builtin_bit_cast(unsigned long long, v);"
             " unsigned lo = __builtin_amdgcn_readlane((int)(unsigned)x, l), hi = __builtin_amdgcn_readlane("
             "(int)(unsigned)(x >> 32), l); return __builtin_bit_cast(real, (unsigned long long)lo |"
             " ((unsigned long long)hi << 32)); }");
    o.line("DEV real rowsum(real v) { v += dpp<0xB1>(v); v += dpp<0x4E>(v); v += dpp<0x141>(v);"
           " v += dpp<0x140>(v); return v; }");
  }
  if (p.radial) emit_radial(o, p);
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

// Row stores of a lane-per-edge kernel (`lane`, `eb` = first edge of the wave's 64, `e0`, `e1`, the
// destination G and a `__shared__ V4 tile[64 * 17]` in scope): the row of `stride` values whose
// expressions are `vals` (padded with zeros) goes to G + (eb + lane - e0) * stride, 64 values at a
// time through the LDS tile, so that the global stores are 16-byte units in which 16 lanes cover
// 256 contiguous bytes of one row.
void emit_staged_rows(Out& o, const Plan& p, std::vector<std::string> vals, int stride) {
  const int per = p.dtype == CGTP_F64 ? 2 : 4;  // values per 16-byte unit
  const int block_vals = 16 * per;             // values per tile column block
  while (int(vals.size()) < stride) vals.push_back("R(0)");
  const int nblocks = (stride + block_vals - 1) / block_vals;
  for (int b = 0; b < nblocks; ++b) {
    const int v0 = b * block_vals, nv = std::min(block_vals, stride - v0) / per;
    o.open("");
    for (int k = 0; k < nv; ++k) {
      std::string v;
      for (int t = 0; t < per; ++t) v += (t ? ", " : "") + vals[size_t(v0 + k * per + t)];
      o.line(F("tile[lane * 17 + %d] = V4{", k) + v + "};");
    }
    o.line("__syncthreads();");
    o.open("for (int it = 0; it < 16; ++it)");
    o.line("const int row = it * 4 + (lane >> 4), c = lane & 15;");
    o.line(F("if (eb + row < e1 && c < %d) ((V4*)(G + (i64)(eb + row - e0) * %d + %d))[c] = tile[row * 17 + c];", nv,
             stride, v0));
    o.close();
    o.line("__syncthreads();");
    o.close();
  }
}

// prep: lane = edge, one wave per 64 edges; writes the G row of every edge of [e0, e1) at
// G + (e - e0) * stride.  Rows are produced 64 values at a time into an LDS tile and copied out
// with 16-byte stores in which 16 lanes cover 256 contiguous bytes of one row.
void emit_prep(Out& o, const Plan& p, bool with_y) {
  const int stride = with_y ? bwd_row_stride(p) : p.g_stride;
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_prep(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, int e0, int e1, real* __restrict__ G)");
  o.line("__shared__ V4 tile[64 * 17];");
  o.line("const int lane = (int)threadIdx.x;");
  o.line("const int eb = e0 + (int)blockIdx.x * 64;");
  o.line("const int e = min(eb + lane, e1 - 1);");
  emit_edge_vector(o);
  o.line("const real rr = sqrt(rx * rx + ry * ry + rz * rz), inv = R(1) / rr;");
  o.line(F("real Y[%d];", p.sh_dim));
  o.line("sh_eval<real>(rx * inv, ry * inv, rz * inv, Y);");
  std::vector<std::string> vals(size_t(p.g_stride), "R(0)");
  if (p.radial) {
    o.line(F("real fr[%d];", p.K));
    o.line("radial_eval(rr, fr, nullptr, nullptr);");
    for (int q = 0; q < p.K; ++q) vals[size_t(p.phi_off + q)] = F("fr[%d]", q);
  }
  for (const Path& P : p.paths) {
    int s = P.l2 * P.l2;
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      std::string ex;
      for (auto& tm : P.gpairs[t].terms) {
        if (!ex.empty()) ex += " + ";
        ex += lit(tm.second) + " * Y[" + std::to_string(s + tm.first) + "]";
      }
      vals[size_t(P.g_off) + t] = ex;
    }
  }
  if (with_y)
    for (int m = 0; m < p.sh_dim; ++m) vals.push_back(F("Y[%d]", m));
  emit_staged_rows(o, p, vals, stride);
  o.close();
}

// Rows of the third-order passes: the folded coefficients G = sum c b and the edge operand b itself
// (the backward's row layout), from an edge operand b given per sorted edge (E x sh_dim) instead of
// the harmonics of the edge vector.  Lane = edge; the same LDS-staged 16-byte row stores as
// cgtp_prep.
void emit_prep_y(Out& o, const Plan& p) {
  const int stride = bwd_row_stride(p);
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_prep_y(const real* __restrict__ yop, int e0, int e1, real* __restrict__ G)");
  o.line("__shared__ V4 tile[64 * 17];");
  o.line("const int lane = (int)threadIdx.x;");
  o.line("const int eb = e0 + (int)blockIdx.x * 64;");
  o.line("const int e = min(eb + lane, e1 - 1);");
  o.line(F("real Y[%d];", p.sh_dim));
  o.line(F("for (int m = 0; m < %d; ++m) Y[m] = yop[(i64)e * %d + m];", p.sh_dim, p.sh_dim));
  std::vector<std::string> vals(size_t(p.g_stride), "R(0)");
  for (const Path& P : p.paths) {
    int s0 = P.l2 * P.l2;
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      std::string ex;
      for (auto& tm : P.gpairs[t].terms) {
        if (!ex.empty()) ex += " + ";
        ex += lit(tm.second) + " * Y[" + std::to_string(s0 + tm.first) + "]";
      }
      vals[size_t(P.g_off) + t] = ex;
    }
  }
  for (int m = 0; m < p.sh_dim; ++m) vals.push_back(F("Y[%d]", m));
  emit_staged_rows(o, p, vals, stride);
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

// Statement `dst (=|+=) G[idx] * xop` with G[idx] taken from its chunk by row broadcast; the
// chunk is loaded on first use.
std::vector<int> chunks_of(const std::vector<std::pair<int, int>>& ranges) {
  std::vector<int> out;
  for (auto& r : ranges)
    for (int c = r.first / 64; r.second > r.first && c <= (r.second - 1) / 64; ++c)
      if (std::find(out.begin(), out.end(), c) == out.end()) out.push_back(c);
  return out;
}

std::vector<std::pair<int, int>> g_ranges(const Plan& p, const std::vector<int>& paths) {
  std::vector<std::pair<int, int>> v;
  for (int pi : paths) v.push_back({p.paths[pi].g_off, p.paths[pi].g_off + int(p.paths[pi].gpairs.size())});
  return v;
}

std::string bcast_term(Out& o, RowChunks& rc, int idx, const std::string& dst, const std::string& xop, bool first) {
  const int c = idx / 64, r = (idx % 64) / 4;
  auto load = [&](int k) {
    if (rc.loaded.insert(k).second)
      o.line(F("const V4 gc%s%d = gchunk(%s, %d, %d, r16_);", rc.tag.c_str(), k, rc.row.c_str(), 64 * k, rc.lim));
  };
  // The first use of each chunk keeps the next kChunkAhead chunks of the list in flight (a sliding
  // window rather than a burst of loads at every chunk not yet loaded).
  if (rc.used.insert(c).second) {
    if (!rc.loaded.count(c)) load(c);
    auto it = std::find(rc.order.begin(), rc.order.end(), c);
    if (it != rc.order.end()) {
      bool ahead = false;
      for (int n = 1; n <= kChunkAhead && it + n < rc.order.end(); ++n)
        if (!rc.loaded.count(*(it + n))) {
          load(*(it + n));
          ahead = true;
        }
      if (ahead) o.line("__builtin_amdgcn_sched_barrier(0);");
    }
  }
  const std::string reg = F("gc%s%d.%c", rc.tag.c_str(), c, "abcd"[idx % 4]);
  if (first) return F("real %s; BMUL(%s, %s, %s, %d);", dst.c_str(), dst.c_str(), reg.c_str(), xop.c_str(), r);
  return F("BFMA(%s, %s, %s, %d);", dst.c_str(), reg.c_str(), xop.c_str(), r);
}

// acc<m3> += w * sum_m1 G[m1,m3] x[m1] for path pi, choosing where to apply w by cost.  The
// accumulators are named <acc><m3>.  With `rc` the coefficients come by row broadcast from
// per-row chunks (each 16-lane row of the wave on its own edge).
void emit_path_accumulate(Out& o, const Plan& p, int pi, const std::string& acc = "acc", RowChunks* rc = nullptr) {
  const Path& P = p.paths[pi];
  const int d1 = 2 * P.l1 + 1, d3 = 2 * P.l3 + 1;
  const char* A = acc.c_str();
  auto G = [&](size_t t) { return gref(p, pi, int(t), "g", "", false); };
  if (d1 <= d3) {
    for (int m = 0; m < d1; ++m) o.line(F("const real s%d_%d = w%d * x%d_%d;", pi, m, pi, P.i_in, m));
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      const int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
      if (rc)
        o.line(bcast_term(o, *rc, P.g_off + int(t), F("%s%d", A, m3), F("s%d_%d", pi, m1), false));
      else
        o.line(F("%s%d = fma(%s, s%d_%d, %s%d);", A, m3, G(t).c_str(), pi, m1, A, m3));
    }
  } else {
    std::vector<bool> started(d3, false);
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
      if (rc)
        o.line(bcast_term(o, *rc, P.g_off + int(t), F("t%d_%d", pi, m3), F("x%d_%d", P.i_in, m1), !started[m3]));
      else if (!started[m3])
        o.line(F("real t%d_%d = %s * x%d_%d;", pi, m3, G(t).c_str(), P.i_in, m1));
      else
        o.line(F("t%d_%d = fma(%s, x%d_%d, t%d_%d);", pi, m3, G(t).c_str(), P.i_in, m1, pi, m3));
      started[m3] = true;
    }
    for (int m = 0; m < d3; ++m)
      if (started[m]) o.line(F("%s%d = fma(w%d, t%d_%d, %s%d);", A, m, pi, pi, m, A, m));
  }
}

const char* kFwdArgs =
    "const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
    " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
    " real* __restrict__ out";

// A coefficients per lane held by one path subset of the conventional forward (K per path; 64-bit
// values take two registers each).  Four paths at K = 8 walk the edge list fastest in both
// precisions: larger subsets lower the occupancy of this latency-bound loop more than they save
// in repeated gathers.
constexpr int kFwdAValues = 32;
constexpr int kSrcSplit = 2;   // waves sharing one sender's edge list in the source backward
constexpr int kRecvGroup = 4;  // receivers (one wave each) per workgroup in the receiver backward

// sr = sum_q phi-bar_q dphi_q/dr at rr (the radial part of the edge-vector gradient is sr r-hat);
// 0 when phi is an input.  `pb` names the phi-bar registers pb0..pb{K-1}.
void emit_radial_term(Out& o, const Plan& p, const std::string& pb) {
  if (!p.radial) {
    o.line("const real sr = R(0);");
    return;
  }
  o.line(F("real fr[%d], dfr[%d];", p.K, p.K));
  o.line("radial_eval(rr, fr, dfr, nullptr);");
  std::string ex = F("%s0 * dfr[0]", pb.c_str());
  for (int q = 1; q < p.K; ++q) ex += F(" + %s%d * dfr[%d]", pb.c_str(), q, q);
  o.line("const real sr = " + ex + ";");
}

// Pointer to the K radial values of the current edge: the phi input, or the edge's G row
// (`grow`) when the plan computes the basis itself.
std::string phi_ptr(const Plan& p, const std::string& e, const std::string& grow) {
  if (p.radial) return F("%s + %d", grow.c_str(), p.phi_off);
  return F("phi + (i64)%s * %d", e.c_str(), p.K);
}

// Loop over the in-edges e0 + start, e0 + start + stride, ... of a receiver (`e0`, `e1` in
// scope).  The rows x_j of the input blocks `blocks` are gathered at the top of each edge's body
// (other waves of the SIMD cover the latency; gathering the next edge's row ahead of the current
// edge's arithmetic measured slower in the forward).  The body sees e, j, g (G row), f<q> (phi)
// and x<b>_<m>.
void emit_recv_edge_loop(Out& o, const Plan& p, const std::vector<int>& blocks, const std::string& start,
                         const std::string& stride, const std::function<void()>& body, bool block_uc,
                         int row_stride, int nE) {
  auto ucn = [&](int b) { return block_uc ? F("uc%d", b) : std::string("uc"); };
  if (row_stride <= 0) row_stride = p.g_stride;
  auto xrow = [&](const char* pre, const char* j, const char* type) {
    for (int b : blocks) {
      const Block& B = p.in[b];
      for (int m = 0; m < B.dim(); ++m)
        o.line(F("%s%s%d_%d = x[(i64)%s * %d + %d + %s];", type, pre, b, m, j, p.c_in, B.offset + m * B.mul,
                 ucn(b).c_str()));
    }
  };
  // The sender indices of up to 64 of the wave's edges are loaded at once, one per lane, and
  // taken one by one with readlane: no scalar-load round trip before each edge's row gather.
  o.open("");
  o.line("const int li_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));");
  o.open("for (int eb_ = e0 + " + start + "; eb_ < e1; eb_ += 64 * " + stride + ")");
  o.line("const int el_ = eb_ + li_ * " + stride + ";");
  o.line("const int cl_ = col[el_ < e1 ? el_ : eb_];");
  o.line("const int ne_ = min(64, (e1 - eb_ + " + stride + " - 1) / " + stride + ");");
  if (nE > 1) {
    // Group h_ of the wave takes edge k_ + h_ of the batch: its sender from lane k_ + h_ of cl_
    // (cl_ holds a valid sender in every lane), its rows and phi by per-lane pointers.
    o.line(F("const int h_ = li_ / %d;", 64 / nE));
    o.open(F("for (int k_ = 0; k_ < ne_; k_ += %d)", nE));
    o.line("const bool ok_ = k_ + h_ < ne_;");
    o.line("const int e = eb_ + (ok_ ? k_ + h_ : k_) * " + stride + ";");
    o.line("const int j = __shfl(cl_, k_ + h_);");
    xrow("x", "j", "const real ");
    o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", row_stride));
    o.line("const real* __restrict__ ph = " + phi_ptr(p, "e", "g") + ";");
    // Loaded unconditionally (e is a valid edge in every lane) and then masked: a load under the
    // condition would become one branch per value.
    for (int q = 0; q < p.K; ++q) o.line(F("const real fl%d_ = ph[%d], f%d = ok_ ? fl%d_ : R(0);", q, q, q, q));
    body();
    o.close();
    o.close();
    o.close();
    return;
  }
  o.open("for (int k_ = 0; k_ < ne_; ++k_)");
  o.line("const int e = eb_ + k_ * " + stride + ";");
  o.line("const int j = __builtin_amdgcn_readlane(cl_, k_);");
  xrow("x", "j", "const real ");
  o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", row_stride));
  o.line("const real* __restrict__ ph = " + phi_ptr(p, "e", "g") + ";");
  for (int q = 0; q < p.K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
  body();
  o.close();
  o.close();
  o.close();
}

// Loop over all in-edges of a receiver (`e0`, `e1` in scope), unrolled by two so that the rows x_j
// prefetched one edge ahead alternate between two register sets (no copies between iterations).
// The body sees e, g (workspace row of `row_stride` values), f<q> (phi) and x<b>_<m>.
void emit_recv_edge_loop2(Out& o, const Plan& p, const std::vector<int>& blocks, int row_stride,
                          const std::function<void()>& body) {
  auto xrow = [&](const char* set) {
    for (int b : blocks) {
      const Block& B = p.in[b];
      for (int m = 0; m < B.dim(); ++m)
        o.line(F("%s%d_%d = x[(i64)jn * %d + %d + uc];", set, b, m, p.c_in, B.offset + m * B.mul));
    }
  };
  auto half = [&](const char* cur, const char* next) {
    o.open("");
    o.line("{ const int en = e + 1; jn = col[en < e1 ? en : e]; }");
    xrow(next);
    for (int b : blocks)
      for (int m = 0; m < p.in[b].dim(); ++m) o.line(F("const real x%d_%d = %s%d_%d;", b, m, cur, b, m));
    o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", row_stride));
    o.line("const real* __restrict__ ph = " + phi_ptr(p, "e", "g") + ";");
    for (int q = 0; q < p.K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
    body();
    o.close();
    o.line("if (++e >= e1) break;");
  };
  o.open("");
  o.line("int e = e0;");
  o.open("if (e < e1)");
  o.line("int jn = col[e];");
  for (int b : blocks)
    for (int m = 0; m < p.in[b].dim(); ++m) o.line(F("real xa%d_%d, xb%d_%d;", b, m, b, m));
  xrow("xa");
  o.open("for (;;)");
  half("xa", "xb");
  half("xb", "xa");
  o.close();
  o.close();
  o.close();
}

// Combine per-wave partial sums acc<m> (m < n) of the waves of a workgroup through LDS in a fixed
// order; afterwards wave 0 holds the total.  `sm` must hold (nw - 1) * n * 64 values.
void emit_wave_combine(Out& o, const std::string& prefix, int n, int nw) {
  if (nw == 1) return;
  o.open("if (w != 0)");
  for (int m = 0; m < n; ++m) o.line(F("sm[((w - 1) * %d + %d) * 64 + lane] = %s%d;", n, m, prefix.c_str(), m));
  o.close();
  o.line("__syncthreads();");
  o.open("if (w == 0)");
  for (int k = 1; k < nw; ++k)
    for (int m = 0; m < n; ++m)
      o.line(F("%s%d += sm[(%d * %d + %d) * 64 + lane];", prefix.c_str(), m, k - 1, n, m));
  o.close();
}

// emit_wave_combine over an explicit list of accumulator names.
void emit_wave_combine_names(Out& o, const std::vector<std::string>& names, int nw) {
  if (nw == 1) return;
  const int n = int(names.size());
  o.open("if (w != 0)");
  for (int m = 0; m < n; ++m) o.line(F("sm[((w - 1) * %d + %d) * 64 + lane] = %s;", n, m, names[m].c_str()));
  o.close();
  o.line("__syncthreads();");
  o.open("if (w == 0)");
  for (int k = 1; k < nw; ++k)
    for (int m = 0; m < n; ++m) o.line(F("%s += sm[(%d * %d + %d) * 64 + lane];", names[m].c_str(), k - 1, n, m));
  o.close();
}

// Channelwise conventional forward of task (output block k, channel block cb) for one receiver;
// the receiver's edges are dealt round-robin to the fwd_split waves of the workgroup and their
// partial sums combined in LDS.  Paths are processed in register-budgeted subsets, each
// re-walking the edges.
// accumulate: add into `out` instead of overwriting it (the third-order passes sum terms there).
// Edges per wave step of the channelwise forward: a block of at most 16 channels fills only a
// quarter of the 64 lanes with one edge, so 4 edges of the receiver share the wave (their
// coefficient rows then come through per-lane loads instead of scalar ones).  Measured: 16
// channels, l <= 3 diamond graph, 99 -> 61 us; two edges of 32-channel blocks measured slower
// (102 -> 109 us at l <= 3, 7.2 -> 9.9 ms at l <= 6: the per-lane row loads cost more than the
// idle half of the lanes), so blocks above 16 channels keep one edge per wave.
int edges_per_wave(int mul) { return mul <= 16 ? 4 : 1; }

// Edges per wave step of the channelwise passes that read coefficient rows per edge: in fp32 each
// 16-lane row takes its coefficients from its own row chunk by row broadcast (one 16-byte load
// per lane serves 64 coefficients), so blocks of at most 32 channels share the wave between 2 or
// 4 edges.  Measured at l <= 6 with 32 channels: forward 7.2 -> 4.1 ms.
int bcast_edges_per_wave(const Plan& p, int mul) {
  if (p.dtype == CGTP_F64) return edges_per_wave(mul);
  return mul <= 16 ? 4 : mul <= 32 ? 2 : 1;
}

void emit_fwd_task(Out& o, const Plan& p, int ti, const Task& T, int row_stride = 0, bool accumulate = false) {
  const int MUL = p.out[p.paths[T.paths[0]].i_out].mul;
  const int nE = bcast_edges_per_wave(p, MUL), gsz = 64 / nE;
  const bool bcast = nE > 1 && p.dtype != CGTP_F64;
  const std::vector<int> obs = out_blocks_of(p, T.paths);
  o.open(F("DEV void fwd_t%d(%s, real* sm, int node, int e_base)", ti, kFwdArgs));
  o.line(F("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) %% %d;",
           fwd_split(p)));
  emit_vz(o, p);
  if (nE > 1)   // channel of the lane inside its edge group
    o.line(F("const int u = lane %% %d;", gsz));
  else
    o.line(F("const int u = %d + lane;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  if (bcast) o.line("const int r16_ = lane & 15;");
  std::vector<std::string> accs;
  for (int ob : obs)
    for (int m = 0; m < p.out[ob].dim(); ++m) {
      accs.push_back(F("acc%d_%d", ob, m));
      o.line("real " + accs.back() + " = R(0);");
    }
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  for (const auto& S : a_subsets(p, T.paths, kFwdAValues * (p.dtype == CGTP_F64 ? 2 : 1))) {
    o.open("");
    emit_a_loads(o, p, S);
    emit_recv_edge_loop(o, p, in_blocks_of(p, S), "w", std::to_string(fwd_split(p)), [&] {
      RowChunks rc{row_stride > 0 ? row_stride : p.g_stride, "g", "", chunks_of(g_ranges(p, S))};
      for (int pi : S) {
        emit_w(o, p, pi);
        emit_path_accumulate(o, p, pi, F("acc%d_", p.paths[pi].i_out), bcast ? &rc : nullptr);
      }
    }, false, row_stride, nE);
    o.close();
  }
  // Edge groups of the wave hold partial sums of the same channels: add them (fixed order).
  for (int span = gsz; span < 64; span *= 2)
    for (const std::string& a : accs) o.line(F("%s += __shfl_xor(%s, %d);", a.c_str(), a.c_str(), span));
  emit_wave_combine_names(o, accs, fwd_split(p));
  o.open(nE > 1 ? F("if (w == 0 && lane < %d && u < %d)", gsz, MUL) : F("if (w == 0 && u < %d)", MUL));
  o.line(F("real* __restrict__ dst = out + (i64)node * %d + u;", p.c_out));
  for (int ob : obs)
    for (int m = 0; m < p.out[ob].dim(); ++m)
      o.line(F(accumulate ? "dst[%d] += acc%d_%d;" : "dst[%d] = acc%d_%d;", p.out[ob].offset + m * MUL, ob, m));
  o.close();
  o.close();
}

// Channelwise streamed forward (Sobek Eqs. 33-34): per path, the receiver state
// S[q][m3] = sum_j phi_q C_pi[m3] over the incoming edges, then m += sum_q S[q] A[q, pi, u].
void emit_fwd_streamed_task(Out& o, const Plan& p, int ti, const Task& T) {
  const Block& OB = p.out[T.group];
  const int d3 = OB.dim(), MUL = OB.mul, K = p.K;
  o.open(F("DEV void fwds_t%d(%s, real* sm, int node, int e_base)", ti, kFwdArgs));
  o.line(F("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) %% %d;",
           fwd_split(p)));
  emit_vz(o, p);
  o.line(F("const int u = %d + lane;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  for (int m = 0; m < d3; ++m) o.line(F("real acc%d = R(0);", m));
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  for (int pi : T.paths) {
    const Path& P = p.paths[pi];
    o.open("");
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d3; ++m) o.line(F("real S%d_%d = R(0);", q, m));
    emit_recv_edge_loop(o, p, {P.i_in}, "w", std::to_string(fwd_split(p)), [&] {
      std::vector<bool> started(d3, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        const std::string G = gref(p, pi, int(t), "g", "", false);
        if (!started[m3])
          o.line(F("real c%d = %s * x%d_%d;", m3, G.c_str(), P.i_in, m1));
        else
          o.line(F("c%d = fma(%s, x%d_%d, c%d);", m3, G.c_str(), P.i_in, m1, m3));
        started[m3] = true;
      }
      for (int q = 0; q < K; ++q)
        for (int m = 0; m < d3; ++m)
          if (started[m]) o.line(F("S%d_%d = fma(f%d, c%d, S%d_%d);", q, m, q, m, q, m));
    });
    for (int q = 0; q < K; ++q) {
      o.line(F("const real a%d = A[%d + uc];", q, q * p.n_w + P.w_off));
      for (int m = 0; m < d3; ++m) o.line(F("acc%d = fma(S%d_%d, a%d, acc%d);", m, q, m, q, m));
    }
    o.close();
  }
  emit_wave_combine(o, "acc", d3, fwd_split(p));
  o.open(F("if (w == 0 && u < %d)", MUL));
  o.line(F("real* __restrict__ dst = out + (i64)node * %d + %d + u;", p.c_out, OB.offset));
  for (int m = 0; m < d3; ++m) o.line(F("dst[%d] = acc%d;", m * MUL, m));
  o.close();
  o.close();
}

int max_out_dim(const Plan& p) {
  int d = 1;
  for (auto& b : p.out) d = std::max(d, b.dim());
  return d;
}

int max_in_dim(const Plan& p) {
  int d = 1;
  for (auto& b : p.in) d = std::max(d, b.dim());
  return d;
}

// One receiver per workgroup of fwd_split waves.  Workgroups are spread over the 8 XCDs
// round-robin by the hardware; this mapping gives each XCD a contiguous receiver range (spatial
// neighbours, whose senders' rows then stay in that XCD's L2) and runs the tasks in decreasing
// cost order inside it (LunaTP section 4.2, task ordering).
// Switch of a grouped dispatch: wave set `cb` of group `t` runs task tasks[t][cb]; the waves of
// a missing channel block only take part in the one workgroup barrier every task function has.
void emit_group_switch(Out& o, const TaskGroups& tg, const std::string& call_fmt, bool barrier) {
  o.open(F("switch (t * %d + cb)", tg.ncb));
  for (int t = 0; t < int(tg.tasks.size()); ++t)
    for (int c = 0; c < int(tg.tasks[t].size()); ++c) {
      std::string call = call_fmt;
      for (size_t at; (at = call.find("%T")) != std::string::npos;) call.replace(at, 2, std::to_string(tg.tasks[t][c]));
      o.line(F("case %d: ", t * tg.ncb + c) + call + " break;");
    }
  o.line(barrier ? "default: __syncthreads(); break;" : "default: break;");
  o.close();
}

void emit_node_dispatch(Out& o, const Plan& p, const std::string& kname, const std::string& args,
                        const std::string& call, const TaskGroups& tg, int nacc) {
  const int slice = (fwd_split(p) - 1) * nacc * 64;
  o.line(F("extern \"C\" __global__ void __launch_bounds__(%d)", 64 * fwd_split(p) * tg.ncb));
  // order (nullable): slot -> receiver of a launch over every node, heaviest first per XCD range.
  o.open(kname + "(" + args + ", int i0, int nrec, int per, int e_base, const int* __restrict__ order)");
  o.line(F("__shared__ real sm[%d];", std::max(1, tg.ncb * slice)));
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, il = s - t * per;");
  o.line("const int i = xcd * per + il;");
  o.line("if (i >= nrec) return;");
  o.line("const int node = order ? order[i] : i0 + i;");
  o.line(F("const int cb = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) / %d;", fwd_split(p)));
  o.line(F("real* const smc = sm + cb * %d;", slice));
  emit_group_switch(o, tg, call + "%T(x, phi, A, G, row_ptr, col, out, smc, node, e_base);", fwd_split(p) > 1);
  o.close();
}

// ------------------------------------------------------------------------------ backward

// Lane swaps of register pairs (a_k, b_k), emitted as inline-assembly blocks: one pair of
// hazard wait states per block instead of per swap.  `width` is 32 or 16.  Registers are
// float or double (a double is swapped as its two 32-bit halves).
void emit_swaps(Out& o, const std::vector<std::pair<std::string, std::string>>& pairs, int width, bool f64) {
  const int kMaxPerBlock = 14;  // 28 asm operands
  std::vector<std::pair<std::string, std::string>> regs;
  if (f64) {
    o.open("");
    for (auto& pr : pairs) {
      for (const std::string* v : {&pr.first, &pr.second}) {
        o.line(F("unsigned long long b_%s = __builtin_bit_cast(unsigned long long, %s);", v->c_str(), v->c_str()));
        o.line(F("unsigned l_%s = (unsigned)b_%s, h_%s = (unsigned)(b_%s >> 32);", v->c_str(), v->c_str(), v->c_str(),
                 v->c_str()));
      }
      regs.push_back({"l_" + pr.first, "l_" + pr.second});
      regs.push_back({"h_" + pr.first, "h_" + pr.second});
    }
  } else {
    regs = pairs;
  }
  for (size_t at = 0; at < regs.size(); at += kMaxPerBlock) {
    size_t n = std::min(regs.size() - at, size_t(kMaxPerBlock));
    std::string text = "s_nop 1\\n\\t";
    std::string ops;
    for (size_t k = 0; k < n; ++k) {
      text += F("v_permlane%d_swap_b32 %%%d, %%%d\\n\\t", width, int(2 * k), int(2 * k + 1));
      ops += F("%s\"+v\"(%s), \"+v\"(%s)", k ? ", " : "", regs[at + k].first.c_str(), regs[at + k].second.c_str());
    }
    text += "s_nop 1";
    o.line("asm volatile(\"" + text + "\" : " + ops + ");");
  }
  if (f64) {
    for (auto& pr : pairs)
      for (const std::string* v : {&pr.first, &pr.second})
        o.line(F("%s = __builtin_bit_cast(real, (unsigned long long)l_%s | ((unsigned long long)h_%s << 32));",
                 v->c_str(), v->c_str(), v->c_str()));
    o.close();
  }
}

// Sums over the 16 lanes of every row of the fp32 registers v0 .. v(n-1), whose row r holds the 16
// partials of one output each, and the stores of the sums.  Instead of a row sum per register
// (four DPP adds each) the registers are transposed pairwise inside the rows: a bank-masked
// row_mirror add puts register 2i's 8-lane partial sums in lanes 0-7 and register 2i+1's in
// lanes 8-15 of register 2i; a row_half_mirror add then merges registers 4j and 4j+2 so that each
// 4-lane bank holds one output (banks 0-3: registers 4j, 4j+2, 4j+1, 4j+3), and two quad
// permutations complete the sums in every lane of the bank: 2 instructions per register where the
// row sums take 4, and one store per four registers.  The DPP adds are inline assembly: each
// group starts with two wait states, so no source was written by a VALU instruction right before,
// and the last one ends with two.  `store(kk, val)` is the statement that stores the sum `val` of
// register `kk` (an int expression) for row r_ = lane >> 4; it runs in the lanes with
// lane & 3 == 0 for which `ok` holds.
void emit_row_reduce_store(Out& o, int n, const std::string& ok,
                           const std::function<std::string(const std::string&, const std::string&)>& store) {
  const int n4 = (n + 3) / 4 * 4;
  // Registers past n exist only as positions: the adds that would fold them are left out (their
  // lanes hold partials of other registers then, and their outputs are never stored).
  auto reg = [&](int k) { return k < n ? F("v%d", k) : std::string(); };
  // One asm group of pair steps: dst = dst + ctrl(dst) on banks m1, dst = src + ctrl(src) on banks
  // m2 (left out without a src).
  auto group = [&](const std::vector<std::array<std::string, 2>>& pairs, const char* ctrl, const char* m1,
                   const char* m2) {
    const size_t kMax = 14;
    for (size_t at = 0; at < pairs.size(); at += kMax) {
      const size_t cnt = std::min(pairs.size() - at, kMax);
      int nsrc = 0;
      for (size_t k = 0; k < cnt; ++k) nsrc += !pairs[at + k][1].empty();
      // outputs %0 .. %(cnt-1): the pairs' first registers; inputs %cnt ..: the second ones
      std::string text, ops, ins;
      for (size_t k = 0, si = 0; k < cnt; ++k) {
        text += F("v_add_f32_dpp %%%d, %%%d, %%%d %s row_mask:0xf bank_mask:%s\\n\\t", int(k), int(k), int(k), ctrl, m1);
        ops += F("%s\"+v\"(%s)", k ? ", " : "", pairs[at + k][0].c_str());
        if (pairs[at + k][1].empty()) continue;
        const int src = int(cnt + si);
        text += F("v_add_f32_dpp %%%d, %%%d, %%%d %s row_mask:0xf bank_mask:%s\\n\\t", int(k), src, src, ctrl, m2);
        ins += F("%s\"v\"(%s)", si ? ", " : "", pairs[at + k][1].c_str());
        ++si;
      }
      o.line("asm volatile(\"s_nop 1\\n\\t" + text + "\" : " + ops + (nsrc ? " : " + ins : "") + ");");
    }
  };
  std::vector<std::array<std::string, 2>> pr;
  for (int i = 0; 2 * i < n; ++i) pr.push_back({reg(2 * i), reg(2 * i + 1)});
  group(pr, "row_mirror", "0x3", "0xc");
  pr.clear();
  for (int j = 0; j < n4 / 4; ++j) pr.push_back({reg(4 * j), reg(4 * j + 2)});
  group(pr, "row_half_mirror", "0x5", "0xa");
  for (const char* qp : {"quad_perm:[1,0,3,2]", "quad_perm:[2,3,0,1]"})
    for (int j0 = 0; j0 < n4 / 4; j0 += 14) {
      std::string t, ops;
      for (int j = j0; j < std::min(n4 / 4, j0 + 14); ++j) {
        t += F("v_add_f32_dpp %%%d, %%%d, %%%d %s row_mask:0xf bank_mask:0xf\\n\\t", j - j0, j - j0, j - j0, qp);
        ops += F("%s\"+v\"(%s)", j > j0 ? ", " : "", reg(4 * j).c_str());
      }
      // the last group ends with two wait states too, before code that does not know its writes
      const bool last = std::string(qp) == "quad_perm:[2,3,0,1]" && j0 + 14 >= n4 / 4;
      o.line("asm volatile(\"s_nop 1\\n\\t" + t + (last ? "s_nop 1" : "") + "\" : " + ops + ");");
    }
  o.open("if ((lane & 3) == 0 && (" + ok + "))");
  o.line("const int r_ = lane >> 4, pb_ = (((lane >> 2) & 1) << 1) | ((lane >> 3) & 1);");
  o.line("(void)r_;");
  for (int j = 0; j < n4 / 4; ++j) {
    o.open("");
    o.line(F("const int kk_ = %d + pb_;", 4 * j));
    o.line(F("if (kk_ < %d) ", n) + store("kk_", reg(4 * j)));
    o.close();
  }
  o.close();
}

void emit_group_reduce_store(Out& o, int V, int nreal, int gsz, bool f64, const std::string& dst_expr) {
  if (!f64) {
    if (gsz == 32) {
      // Columns k and k + V/2 of the two 32-lane halves: one permlane16 swap puts column k of edge
      // A, column k + V/2 of A, k of B and k + V/2 of B in rows 0..3 of register k.
      const int H = V / 2;
      std::vector<std::pair<std::string, std::string>> pr;
      for (int k = 0; k < H; ++k) pr.push_back({F("v%d", k), F("v%d", k + H)});
      emit_swaps(o, pr, 16, false);
      for (int k = 0; k < H; ++k) o.line(F("v%d += v%d;", k, k + H));
      emit_row_reduce_store(o, H, "ok_", [&](const std::string& kk, const std::string& val) {
        return "(" + dst_expr + F(")[64 * (%s + (r_ & 1) * %d)] = %s;", kk.c_str(), H, val.c_str());
      });
    } else {   // one edge per row, its columns in v0 .. v(nreal - 1) (the rest are padding, zero)
      emit_row_reduce_store(o, nreal, "ok_", [&](const std::string& kk, const std::string& val) {
        return "(" + dst_expr + ")[64 * " + kk + "] = " + val + ";";
      });
    }
    return;
  }
  if (gsz == 32) {
    // Columns k and k + V/2 of the two 32-lane halves: one permlane16 swap puts column k of edge A,
    // column k + V/2 of A, k of B and k + V/2 of B in rows 0..3, each row holding 16 lanes' worth
    // of both rows of its half; one row sum then completes all four.
    const int H = V / 2;
    std::vector<std::pair<std::string, std::string>> pr;
    for (int k = 0; k < H; ++k) pr.push_back({F("v%d", k), F("v%d", k + H)});
    emit_swaps(o, pr, 16, f64);
    for (int k = 0; k < H; ++k) o.line(F("v%d += v%d;", k, k + H));
    for (int k = 0; k < H; ++k) o.line(F("v%d = rowsum(v%d); asm volatile(\"\" : \"+v\"(v%d));", k, k, k));
    o.open("if ((lane & 15) == 0 && ok_)");
    o.line("real* __restrict__ dst = " + dst_expr + " + ((lane >> 4) & 1) * " + std::to_string(64 * H) + ";");
    for (int k = 0; k < H; ++k) o.line(F("dst[%d] = v%d;", 64 * k, k));
    o.close();
    return;
  }
  for (int k = 0; k < V; ++k) o.line(F("v%d = rowsum(v%d); asm volatile(\"\" : \"+v\"(v%d));", k, k, k));
  o.open(F("if ((lane & %d) == 0 && ok_)", gsz - 1));
  o.line("real* __restrict__ dst = " + dst_expr + ";");
  for (int k = 0; k < V; ++k) o.line(F("dst[%d] = v%d;", 64 * k, k));
  o.close();
}

const char* kRecvArgs =
    "const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ A,"
    " const real* __restrict__ G, const int* __restrict__ row_ptr, const int* __restrict__ col,"
    " const real* __restrict__ gout, real* __restrict__ ep, real* __restrict__ ap";

// (m1, m2) pairs of a path's CG tensor with their (m3, c) terms: R[m1, m2] = sum_m3 c mbar[m3].
std::vector<std::pair<std::pair<int, int>, std::vector<std::pair<int, double>>>> m12_pairs(const Path& P) {
  std::vector<std::pair<std::pair<int, int>, std::vector<std::pair<int, double>>>> v;
  for (const CGTerm& t : P.terms) {
    std::pair<int, int> key{t.m1, t.m2};
    auto it = std::find_if(v.begin(), v.end(), [&](const auto& e) { return e.first == key; });
    if (it == v.end()) {
      v.push_back({key, {}});
      it = v.end() - 1;
    }
    it->second.push_back({t.m3, t.c});
  }
  return v;
}

// A path of the receiver backward runs in "receiver-folded" form when its (m1, m2) table fits the
// register budget: R = sum_m3 c mbar[m3] is formed once per receiver, and per edge
// Q[m2] = sum_m1 x[m1] R[m1, m2] gives both h = sum_m2 Y[m2] Q[m2] (Eq. 18) and the Y-bar
// partials w Q[m2] (Eq. 22) without forming T = G x.
constexpr int kFoldMax = 48;     // largest (m1, m2) table kept in registers
constexpr int kRecvBudget = 176;  // registers per lane for A, the A-bar accumulators and R of one task
// Plans with large paths (vector coefficient loads): streamed rows and kRecvLargeDiv times smaller
// tasks in the receiver backward.
constexpr bool kRecvStreamLarge = true;
constexpr int kRecvLargeDiv = 4;

bool folded(const Path& P) { return int(m12_pairs(P).size()) <= kFoldMax; }

// Receiver-major backward of task (output block k, path subset, channel block) for one receiver
// per wave (node < 0: no receiver).  Per edge: h_pi = <mbar, T_pi> (Eq. 18), phi-bar partials
// sum_pi A h (Eq. 20) and Y-bar partials sum_pi w sum c x mbar (Eq. 22), reduced over the 64
// channels of the wave and stored in slot `ti` of the edge's partial column.  A-bar = sum_e phi h
// (Eq. 19) accumulates in registers, is combined over the kRecvGroup waves of the workgroup in
// LDS and added to the workgroup's partial slot.  Folded paths read Y from the edge's workspace
// row (after the G values); the others contract G as in the forward.
void emit_bwd_recv_task(Out& o, const Plan& p, int ti, const Task& T, int col_off, int row) {
  const int MUL = p.out[p.paths[T.paths[0]].i_out].mul, K = p.K;
  const std::vector<int> ycols = recv_task_ycols(p, T);
  const int V = recv_task_width(p, T);
  auto ycol = [&](int y) { return K + int(std::find(ycols.begin(), ycols.end(), y) - ycols.begin()); };
  // Blocks of at most 16 (32) channels: 4 (2) edges per wave step, one per 16-lane row (32-lane
  // half); the per-edge channel reductions are then row sums (and one add across the two rows of a
  // half) instead of the 64-lane transposition, and each group stores its own edge's columns.  The
  // rows this pass reads per edge are short (Y, or large paths' coefficients already read per lane),
  // so unlike the forward the 32-channel case gains too.
  // In fp32 each row takes its edge's coefficients and Y values by row broadcast.
  const int nE = MUL <= 16 ? 4 : MUL <= 32 ? 2 : 1, gsz = 64 / nE;
  const bool bcast = nE > 1 && p.dtype != CGTP_F64;
  o.open(F("DEV void bwr_t%d(%s, real* sm, int node, int e_base, int eps, int slot, int acc)", ti, kRecvArgs));
  o.line("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  if (bcast) o.line("const int r16_ = lane & 15;");
  emit_vz(o, p);
  if (nE > 1)
    o.line(F("const int u = lane %% %d;", gsz));
  else
    o.line(F("const int u = %d + lane;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  emit_a_loads(o, p, T.paths);
  std::vector<std::string> aa;  // A-bar accumulators: K per path of the task
  for (size_t n = 0; n < T.paths.size() * size_t(K); ++n) {
    o.line(F("real aa%d = R(0);", int(aa.size())));
    aa.push_back(F("aa%d", int(aa.size())));
  }
  o.open("if (node >= 0)");
  o.line(F("const real* __restrict__ gr = gout + (i64)node * %d + uc;", p.c_out));
  for (int ob : out_blocks_of(p, T.paths)) {
    const Block& OB = p.out[ob];
    for (int m = 0; m < OB.dim(); ++m)
      o.line(F("const real mb%d_%d = u < %d ? gr[%d] : R(0);", ob, m, MUL, OB.offset + m * MUL));
  }
  for (int pi : T.paths) {
    const Path& P = p.paths[pi];
    if (!folded(P)) continue;
    for (auto& pr : m12_pairs(P)) {
      std::string ex;
      for (auto& t : pr.second)
        ex += (ex.empty() ? "" : " + ") + lit(t.second) + F(" * mb%d_%d", P.i_out, t.first);
      o.line(F("const real r%d_%d_%d = ", pi, pr.first.first, pr.first.second) + ex + ";");
    }
  }
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  const int yoff = p.g_stride;  // Y values follow the G values in a workspace row
  auto body = [&] {
    for (int v = 0; v < V; ++v) o.line(F("real v%d = R(0);", v));
    int ai = 0;
    std::vector<std::pair<int, int>> ranges;   // Y values of folded paths, G rows of the others
    for (int pi : T.paths) {
      const Path& P = p.paths[pi];
      if (folded(P)) ranges.push_back({yoff + P.l2 * P.l2, yoff + (P.l2 + 1) * (P.l2 + 1)});
      else ranges.push_back({P.g_off, P.g_off + int(P.gpairs.size())});
    }
    RowChunks rc{bwd_row_stride(p), "g", "", chunks_of(ranges)};
    for (int pi : T.paths) {
      const Path& P = p.paths[pi];
      const int s = K + P.l2 * P.l2;  // Y-bar slot of this path's SH block
      const int d2 = 2 * P.l2 + 1;
      emit_w(o, p, pi);
      if (folded(P)) {
        std::vector<bool> qs(d2, false);
        for (auto& pr : m12_pairs(P)) {
          int m1 = pr.first.first, m2 = pr.first.second;
          if (!qs[m2]) o.line(F("real q%d_%d = x%d_%d * r%d_%d_%d;", pi, m2, P.i_in, m1, pi, m1, m2));
          else o.line(F("q%d_%d = fma(x%d_%d, r%d_%d_%d, q%d_%d);", pi, m2, P.i_in, m1, pi, m1, m2, pi, m2));
          qs[m2] = true;
        }
        bool first = true;
        for (int m = 0; m < d2; ++m)
          if (qs[m]) {
            if (bcast) o.line(bcast_term(o, rc, yoff + P.l2 * P.l2 + m, F("h%d", pi), F("q%d_%d", pi, m), first));
            else if (first) o.line(F("real h%d = g[%d] * q%d_%d;", pi, yoff + P.l2 * P.l2 + m, pi, m));
            else o.line(F("h%d = fma(g[%d], q%d_%d, h%d);", pi, yoff + P.l2 * P.l2 + m, pi, m, pi));
            first = false;
          }
        for (int q = 0; q < K; ++q, ++ai) {
          o.line(F("aa%d = fma(f%d, h%d, aa%d);", ai, q, pi, ai));
          o.line(F("v%d = fma(a%d_%d, h%d, v%d);", q, pi, q, pi, q));
        }
        for (int m = 0; m < d2; ++m)
          if (qs[m]) o.line(F("v%d = fma(w%d, q%d_%d, v%d);", ycol(s - K + m), pi, pi, m, ycol(s - K + m)));
        continue;
      }
      const int d3 = 2 * P.l3 + 1, ob = P.i_out;
      std::unique_ptr<GStream> gs;
      if (!bcast) gs.reset(new GStream(o, p, pi, "g", "", p.vec_g && kRecvStreamLarge));
      std::vector<bool> started(d3, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (bcast) {
          o.line(bcast_term(o, rc, P.g_off + int(t), F("t%d_%d", pi, m3), F("x%d_%d", P.i_in, m1), !started[m3]));
          started[m3] = true;
          continue;
        }
        const std::string G = gs->ref(int(t));
        if (!started[m3])
          o.line(F("real t%d_%d = %s * x%d_%d;", pi, m3, G.c_str(), P.i_in, m1));
        else
          o.line(F("t%d_%d = fma(%s, x%d_%d, t%d_%d);", pi, m3, G.c_str(), P.i_in, m1, pi, m3));
        started[m3] = true;
      }
      bool first = true;
      for (int m = 0; m < d3; ++m)
        if (started[m]) {
          if (first) o.line(F("real h%d = mb%d_%d * t%d_%d;", pi, ob, m, pi, m));
          else o.line(F("h%d = fma(mb%d_%d, t%d_%d, h%d);", pi, ob, m, pi, m, pi));
          first = false;
        }
      for (int q = 0; q < K; ++q, ++ai) {
        o.line(F("aa%d = fma(f%d, h%d, aa%d);", ai, q, pi, ai));
        o.line(F("v%d = fma(a%d_%d, h%d, v%d);", q, pi, q, pi, q));
      }
      std::set<int> m3used;
      for (auto& gp : P.gpairs) m3used.insert(gp.m3);
      for (int m : m3used) o.line(F("const real wm%d_%d = w%d * mb%d_%d;", pi, m, pi, ob, m));
      for (auto& gp : P.gpairs) {
        o.line(F("{ const real z = x%d_%d * wm%d_%d;", P.i_in, gp.m1, pi, gp.m3));
        for (auto& t : gp.terms)
          o.line(F("  v%d = fma(%s, z, v%d);", ycol(s - K + t.first), lit(t.second).c_str(), ycol(s - K + t.first)));
        o.line("}");
      }
    }
    if (nE > 1) {   // one edge per group: its columns reduced over the group's lanes and stored
      emit_group_reduce_store(o, V, K + int(ycols.size()), gsz, p.dtype == CGTP_F64,
                              F("ep + ((i64)((e - e_base) >> 6) * %d + %d) * 64 + ((e - e_base) & 63)", row, col_off));
      return;
    }
    // Transpose-reduce the V partial sums over the 64 lanes: afterwards lane group r = lane / 16
    // holds columns r Q .. r Q + Q - 1 in v0 .. v(Q-1).  The empty asm keeps the row sums in all
    // lanes, so that their last DPP step is not moved under the store's lane mask.
    const int H = V / 2, Q = V / 4;
    const bool f64 = p.dtype == CGTP_F64;
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
  };
  if (nE > 1)
    emit_recv_edge_loop(o, p, in_blocks_of(p, T.paths), "0", "1", body, false, bwd_row_stride(p), nE);
  else
    emit_recv_edge_loop2(o, p, in_blocks_of(p, T.paths), bwd_row_stride(p), body);
  for (int span = gsz; span < 64; span *= 2)
    for (const std::string& a : aa) o.line(F("%s += __shfl_xor(%s, %d);", a.c_str(), a.c_str(), span));
  o.close();  // node >= 0
  emit_wave_combine(o, "aa", int(aa.size()), kRecvGroup);
  o.open(nE > 1 ? F("if (w == 0 && lane < %d && u < %d)", gsz, MUL) : F("if (w == 0 && u < %d)", MUL));
  o.line(F("real* __restrict__ dst = ap + (i64)slot * %d + u;", K * p.n_w));
  // acc = 0 (a single receiver chunk): the slot is written, not accumulated, so it needs no
  // zero fill; every slot's workgroup runs, with node = -1 for missing receivers.
  int ai = 0;
  for (int pi : T.paths)
    for (int q = 0; q < K; ++q, ++ai)
      o.line(F("dst[%d] = acc ? dst[%d] + aa%d : aa%d;", q * p.n_w + p.paths[pi].w_off,
               q * p.n_w + p.paths[pi].w_off, ai, ai));
  o.close();
  o.close();
}

// kRecvGroup consecutive receivers (one wave each) per workgroup: block b -> XCD b & 7, and
// inside it (task, group of receivers); the group is the A-bar partial slot.
void emit_recv_dispatch(Out& o, const Plan& p, int ntask) {
  int amax = 0;
  for (const Task& t : recv_backward_tasks(p)) amax = std::max(amax, int(t.paths.size()) * p.K);
  o.line(F("extern \"C\" __global__ void __launch_bounds__(%d)", 64 * kRecvGroup));
  o.open(std::string("cgtp_bwd_recv(") + kRecvArgs +
         ", int i0, int nrec, int per, int nch, int e_base, int eps, int acc, const int* __restrict__ order)");
  o.line(F("__shared__ real sm[%d];", (kRecvGroup - 1) * amax * 64));
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / nch, c = s - t * nch;");
  o.line(F("const int lo = xcd * per + c * %d;", kRecvGroup));
  o.line(F("int hi = lo + %d; if (hi > (xcd + 1) * per) hi = (xcd + 1) * per; if (hi > nrec) hi = nrec;", kRecvGroup));
  o.line("if (lo >= hi && acc) return;");
  o.line("const int r = lo + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  o.line("const int node = r < hi ? (order ? order[r] : i0 + r) : -1;");
  o.line("const int slot = xcd * nch + c;");
  o.open("switch (t)");
  for (int k = 0; k < ntask; ++k)
    o.line(F("case %d: bwr_t%d(x, phi, A, G, row_ptr, col, gout, ep, ap, sm, node, e_base, eps, slot, acc); break;", k,
             k));
  o.line("default: break;");
  o.close();
  o.close();
}

const char* kSrcArgs =
    "const real* __restrict__ phi, const real* __restrict__ A, const real* __restrict__ G,"
    " const real* __restrict__ gout, const int* __restrict__ recv, const int* __restrict__ src_beg,"
    " const int* __restrict__ src_end, const int* __restrict__ src_edge, real* __restrict__ gx";

// Source-major x-bar of task (input block b, channel block cb) for one sender (Eq. 21):
// x-bar_j[m1] = sum over out-edges, paths of w_pi sum_m3 G[m1,m3] mbar_i[m3].  The out-edges are
// dealt round-robin to the kSrcSplit waves of the workgroup (partials combined in LDS); the
// receivers' mbar rows of the next edge are loaded one edge ahead.
void emit_bwd_src_task(Out& o, const Plan& p, int ti, const Task& T) {
  const int MUL = p.in[p.paths[T.paths[0]].i_in].mul, K = p.K;
  // Blocks of at most 32 channels: 2 or 4 out-edges per wave step, one per lane group (as the forward).
  const int nE = bcast_edges_per_wave(p, MUL), gsz = 64 / nE;
  const bool bcast = nE > 1 && p.dtype != CGTP_F64;
  const std::vector<int> ibs = in_blocks_of(p, T.paths);
  o.open(F("DEV void bws_t%d(%s, real* sm, int node, int e_base, int accumulate)", ti, kSrcArgs));
  o.line(F("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) %% %d;",
           kSrcSplit));
  emit_vz(o, p);
  if (nE > 1)
    o.line(F("const int u = lane %% %d, h_ = lane / %d;", gsz, gsz));
  else
    o.line(F("const int u = %d + lane;", T.cb * 64));
  o.line(F("const int uc = u < %d ? u : %d;", MUL, MUL - 1));
  if (bcast) o.line("const int r16_ = lane & 15;");
  std::vector<std::string> accs;
  for (int ib : ibs)
    for (int m = 0; m < p.in[ib].dim(); ++m) {
      accs.push_back(F("acc%d_%d", ib, m));
      o.line("real " + accs.back() + " = R(0);");
    }
  o.line("const int s0 = src_beg[node], s1 = src_end[node];");
  for (const auto& S : a_subsets(p, T.paths, kRegBudget)) {
  o.open("");
  emit_a_loads(o, p, S);
  const auto obs = out_blocks_of(p, S);
  auto mrow = [&](const char* pre, const char* i, const char* type) {
    for (int ob : obs) {
      const Block& B = p.out[ob];
      for (int m = 0; m < B.dim(); ++m)
        o.line(F("%s%s%d_%d = gout[(i64)%s * %d + %d + uc];", type, pre, ob, m, i, p.c_out, B.offset + m * B.mul));
    }
  };
  // Edge ids and their receivers for up to 64 of the wave's out-edges, one per lane, taken one
  // by one with readlane (no dependent scalar loads before each edge's gather).
  o.open(F("for (int kb_ = s0 + w; kb_ < s1; kb_ += %d)", 64 * kSrcSplit));
  o.line(F("const int kl_ = kb_ + lane * %d;", kSrcSplit));
  o.line("const int el_ = src_edge[kl_ < s1 ? kl_ : kb_];");
  o.line("const int il_ = recv[el_];");
  o.line(F("const int ne_ = min(64, (s1 - kb_ + %d) / %d);", kSrcSplit - 1, kSrcSplit));
  if (nE > 1) {   // group h_ takes out-edge k_ + h_ (el_, il_ hold valid ids in every lane)
    o.open(F("for (int k_ = 0; k_ < ne_; k_ += %d)", nE));
    o.line("const bool ok_ = k_ + h_ < ne_;");
    o.line("const int e = __shfl(el_, k_ + h_);");
    o.line("const int i_ = __shfl(il_, k_ + h_);");
  } else {
    o.open("for (int k_ = 0; k_ < ne_; ++k_)");
    o.line("const int e = __builtin_amdgcn_readlane(el_, k_);");
    o.line("const int i_ = __builtin_amdgcn_readlane(il_, k_);");
  }
  mrow("mb", "i_", "const real ");
  o.line(F("const real* __restrict__ g = G + (i64)(e - e_base) * %d;", bwd_row_stride(p)));
  o.line("const real* __restrict__ ph = " + phi_ptr(p, "e", "g") + ";");
  for (int q = 0; q < K; ++q)
    o.line(nE > 1 ? F("const real fl%d_ = ph[%d], f%d = ok_ ? fl%d_ : R(0);", q, q, q, q)
                  : F("const real f%d = ph[%d];", q, q));
  RowChunks rc{bwd_row_stride(p), "g", "", chunks_of(g_ranges(p, S))};
  for (int pi : S) {
    const Path& P = p.paths[pi];
    const int d1 = 2 * P.l1 + 1, d3 = 2 * P.l3 + 1, ib = P.i_in;
    emit_w(o, p, pi);
    auto G = [&](size_t t) { return gref(p, pi, int(t), "g", "", false); };
    if (d3 <= d1) {
      for (int m = 0; m < d3; ++m) o.line(F("const real s%d_%d = w%d * mb%d_%d;", pi, m, pi, P.i_out, m));
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        const int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (bcast)
          o.line(bcast_term(o, rc, P.g_off + int(t), F("acc%d_%d", ib, m1), F("s%d_%d", pi, m3), false));
        else
          o.line(F("acc%d_%d = fma(%s, s%d_%d, acc%d_%d);", ib, m1, G(t).c_str(), pi, m3, ib, m1));
      }
    } else {
      std::vector<bool> started(d1, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (bcast)
          o.line(bcast_term(o, rc, P.g_off + int(t), F("b%d_%d", pi, m1), F("mb%d_%d", P.i_out, m3), !started[m1]));
        else if (!started[m1])
          o.line(F("real b%d_%d = %s * mb%d_%d;", pi, m1, G(t).c_str(), P.i_out, m3));
        else
          o.line(F("b%d_%d = fma(%s, mb%d_%d, b%d_%d);", pi, m1, G(t).c_str(), P.i_out, m3, pi, m1));
        started[m1] = true;
      }
      for (int m = 0; m < d1; ++m)
        if (started[m]) o.line(F("acc%d_%d = fma(w%d, b%d_%d, acc%d_%d);", ib, m, pi, pi, m, ib, m));
    }
  }
  o.close();
  o.close();
  o.close();
  }
  for (int span = gsz; span < 64; span *= 2)
    for (const std::string& a : accs) o.line(F("%s += __shfl_xor(%s, %d);", a.c_str(), a.c_str(), span));
  emit_wave_combine_names(o, accs, kSrcSplit);
  o.open(nE > 1 ? F("if (w == 0 && lane < %d && u < %d)", gsz, MUL) : F("if (w == 0 && u < %d)", MUL));
  o.line(F("real* __restrict__ dst = gx + (i64)node * %d + u;", p.c_in));
  o.open("if (accumulate)");
  for (int ib : ibs)
    for (int m = 0; m < p.in[ib].dim(); ++m) o.line(F("dst[%d] += acc%d_%d;", p.in[ib].offset + m * MUL, ib, m));
  o.close("} else {");
  ++o.ind;
  for (int ib : ibs)
    for (int m = 0; m < p.in[ib].dim(); ++m) o.line(F("dst[%d] = acc%d_%d;", p.in[ib].offset + m * MUL, ib, m));
  o.close();
  o.close();
  o.close();
}

void emit_src_dispatch(Out& o, const Plan& p, int ntask) {
  int nacc = 1;
  for (const Task& t : source_tasks(p)) {
    int n = 0;
    for (int ib : in_blocks_of(p, t.paths)) n += p.in[ib].dim();
    nacc = std::max(nacc, n);
  }
  const TaskGroups tg = task_groups(source_tasks(p));
  (void)ntask;
  const int slice = (kSrcSplit - 1) * nacc * 64;
  o.line(F("extern \"C\" __global__ void __launch_bounds__(%d)", 64 * kSrcSplit * tg.ncb));
  o.open(std::string("cgtp_bwd_src(") + kSrcArgs +
         ", int nrec, int per, int e_base, int accumulate, const int* __restrict__ order)");
  o.line(F("__shared__ real sm[%d];", std::max(1, tg.ncb * slice)));
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, il = s - t * per;");
  o.line("const int slot = xcd * per + il;");
  o.line("if (slot >= nrec) return;");
  o.line("const int node = order ? order[slot] : slot;");
  o.line(F("const int cb = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) / %d;", kSrcSplit));
  o.line(F("real* const smc = sm + cb * %d;", slice));
  emit_group_switch(o, tg, "bws_t%T(phi, A, G, gout, recv, src_beg, src_end, src_edge, gx, smc, node, e_base, accumulate);",
                    kSrcSplit > 1);
  o.close();
}

// Per-edge finalisation: phi-bar and Y-bar = fixed-order sums of the task partials, then the
// edge-vector gradient e-bar = J_Y(r)^T Y-bar with J_Y = (I - n n^T) dY/dn / |r|.
void emit_edge_final(Out& o, const Plan& p, int ntask, int V) {
  const int K = p.K;
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_edge_final(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ ep, int e0, int e1, int eps,"
         " real* __restrict__ gphi, real* __restrict__ gev)");
  o.line("const int e = e0 + (int)(blockIdx.x * 256 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  o.line("const real* __restrict__ col0 = ep + (e - e0);");
  o.line("#define ROWV(k) col0[(i64)(k) * eps]");
  for (int q = 0; q < K; ++q) {
    std::string ex = F("ROWV(%d)", q);
    for (int t = 1; t < ntask; ++t) ex += F(" + ROWV(%d)", t * V + q);
    o.line(F("const real pb%d = ", q) + ex + ";");
  }
  o.open("if (gphi)");
  for (int q = 0; q < K; ++q) o.line(F("gphi[(i64)e * %d + %d] = pb%d;", K, q, q));
  o.close();
  o.line("if (!gev) return;");
  emit_edge_vector(o);
  o.line("const real rr = sqrt(rx * rx + ry * ry + rz * rz), inv = R(1) / rr;");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line(F("D3 Y[%d];", p.sh_dim));
  o.line("sh_eval<D3>(D3(nx, R(1), R(0), R(0)), D3(ny, R(0), R(1), R(0)), D3(nz, R(0), R(0), R(1)), Y);");
  o.line("real gx = R(0), gy = R(0), gz = R(0);");
  for (int m = 0; m < p.sh_dim; ++m) {
    std::string ex = F("ROWV(%d)", K + m);
    for (int t = 1; t < ntask; ++t) ex += F(" + ROWV(%d)", t * V + K + m);
    o.line(F("{ const real yb = ") + ex + F("; gx = fma(yb, Y[%d].x, gx); gy = fma(yb, Y[%d].y, gy);"
                                             " gz = fma(yb, Y[%d].z, gz); }", m, m, m));
  }
  o.line("const real d = nx * gx + ny * gy + nz * gz;");
  emit_radial_term(o, p, "pb");
  o.line("gev[3 * (i64)e] = (gx - nx * d) * inv + sr * nx;");
  o.line("gev[3 * (i64)e + 1] = (gy - ny * d) * inv + sr * ny;");
  o.line("gev[3 * (i64)e + 2] = (gz - nz * d) * inv + sr * nz;");
  o.line("#undef ROWV");
  o.close();
}

// Edge finalisation of the channelwise backward: the edge's partial row holds, task after task,
// K phi-bar partials and the task's Y-bar columns; sums run over the tasks in a fixed order, then
// e-bar = J_Y(r)^T Y-bar with J_Y = (I - n n^T) dY/dn / |r|.  Partial rows are stored in tiles of
// 64 edges, column-major inside a tile: column c of edge e sits at
// ((e / 64) row + c) 64 + e mod 64, so that both the receiver pass (one base address, immediate
// offsets) and this kernel (lane = edge) access them contiguously.
void emit_recv_edge_final(Out& o, const Plan& p, const std::vector<Task>& tasks) {
  const int K = p.K, row = recv_partial_row(p);
  std::vector<int> off;
  for (int k = 0, c = 0; k < int(tasks.size()); c += recv_task_width(p, tasks[k]), ++k) off.push_back(c);
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_edge_final(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const real* __restrict__ ep, int e0, int e1, int eps,"
         " real* __restrict__ gphi, real* __restrict__ gev)");
  o.line("(void)eps;");
  o.line("const int e = e0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  o.line(F("const real* __restrict__ rw = ep + (i64)((e - e0) >> 6) * %d + ((e - e0) & 63);", 64 * row));
  o.line("#define RW(c) rw[64 * (c)]");
  for (int q = 0; q < K; ++q) {
    std::string ex;
    for (size_t t = 0; t < tasks.size(); ++t) ex += (t ? " + " : "") + F("RW(%d)", off[t] + q);
    o.line(F("const real pb%d = ", q) + ex + ";");
  }
  o.open("if (gphi)");
  for (int q = 0; q < K; ++q) o.line(F("gphi[(i64)e * %d + %d] = pb%d;", K, q, q));
  o.close();
  o.line("if (!gev) return;");
  emit_edge_vector(o);
  o.line("const real rr = sqrt(rx * rx + ry * ry + rz * rz), inv = R(1) / rr;");
  o.line("const real nx = rx * inv, ny = ry * inv, nz = rz * inv;");
  o.line(F("D3 Y[%d];", p.sh_dim));
  o.line("sh_eval<D3>(D3(nx, R(1), R(0), R(0)), D3(ny, R(0), R(1), R(0)), D3(nz, R(0), R(0), R(1)), Y);");
  o.line("real gx = R(0), gy = R(0), gz = R(0);");
  std::vector<std::vector<int>> yc;
  for (const Task& t : tasks) yc.push_back(recv_task_ycols(p, t));
  for (int m = 0; m < p.sh_dim; ++m) {
    std::string ex;
    for (size_t t = 0; t < tasks.size(); ++t) {
      auto it = std::find(yc[t].begin(), yc[t].end(), m);
      if (it == yc[t].end()) continue;
      ex += (ex.empty() ? "" : " + ") + F("RW(%d)", off[t] + K + int(it - yc[t].begin()));
    }
    if (ex.empty()) continue;
    o.line(F("{ const real yb = ") + ex + F("; gx = fma(yb, Y[%d].x, gx); gy = fma(yb, Y[%d].y, gy);"
                                           " gz = fma(yb, Y[%d].z, gz); }", m, m, m));
  }
  o.line("const real d = nx * gx + ny * gy + nz * gz;");
  emit_radial_term(o, p, "pb");
  o.line("gev[3 * (i64)e] = (gx - nx * d) * inv + sr * nx;");
  o.line("gev[3 * (i64)e + 1] = (gy - ny * d) * inv + sr * ny;");
  o.line("gev[3 * (i64)e + 2] = (gz - nz * d) * inv + sr * nz;");
  o.line("#undef RW");
  o.close();
}

// Per-edge finalisation of the third-order passes: phi-bar (K values) and the edge-operand
// gradient Y-bar (sh_dim values) as fixed-order sums of the receiver pass's task partials, written
// for the chunk's edges (rows e - e0).
void emit_recv_edge_final_y(Out& o, const Plan& p, const std::vector<Task>& tasks, bool stacked) {
  const int K = p.K, row = recv_partial_row(p);
  std::vector<int> off;
  for (int k = 0, c = 0; k < int(tasks.size()); c += recv_task_width(p, tasks[k]), ++k) off.push_back(c);
  // Added into the destinations (rows e - e0): with stacked factors phi-bar columns 0 .. K/2 - 1
  // into gphi1 and K/2 .. K - 1 into gphi2 (the derivatives for the two radial factors), else all
  // K columns into gphi1; Y-bar into gy; each nullable.
  const int Kh = stacked ? K / 2 : K;
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_edge_final_y(const real* __restrict__ ep, int e0, int e1, real* __restrict__ gphi1,"
         " real* __restrict__ gphi2, real* __restrict__ gy)");
  o.line("const int e = e0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (e >= e1) return;");
  o.line(F("const real* __restrict__ rw = ep + (i64)((e - e0) >> 6) * %d + ((e - e0) & 63);", 64 * row));
  o.line("#define RW(c) rw[64 * (c)]");
  if (!stacked) o.line("(void)gphi2;");
  for (int h = 0; h < (stacked ? 2 : 1); ++h) {
    o.open(F("if (gphi%d)", h + 1));
    for (int q = h * Kh; q < (h + 1) * Kh; ++q) {
      std::string ex;
      for (size_t t = 0; t < tasks.size(); ++t) ex += (t ? " + " : "") + F("RW(%d)", off[t] + q);
      o.line(F("gphi%d[(i64)(e - e0) * %d + %d] += ", h + 1, Kh, q - h * Kh) + ex + ";");
    }
    o.close();
  }
  o.open("if (gy)");
  std::vector<std::vector<int>> yc;
  for (const Task& t : tasks) yc.push_back(recv_task_ycols(p, t));
  for (int m = 0; m < p.sh_dim; ++m) {
    std::string ex;
    for (size_t t = 0; t < tasks.size(); ++t) {
      auto it = std::find(yc[t].begin(), yc[t].end(), m);
      if (it == yc[t].end()) continue;
      ex += (ex.empty() ? "" : " + ") + F("RW(%d)", off[t] + K + int(it - yc[t].begin()));
    }
    if (!ex.empty()) o.line(F("gy[(i64)(e - e0) * %d + %d] += ", p.sh_dim, m) + ex + ";");
  }
  o.close();
  o.line("#undef RW");
  o.close();
}

// Operand packing and A-bar reduction of the third-order passes.  Their kernels are generated for
// 2K radial values, so that a weight phi_1 A_1 + phi_2 A_2 is one product of the stacked
// [phi_1 | phi_2] (E x 2K) and [A_1; A_2] (2K x N_w); a missing factor is zero.
// stacked false (the plan's own K, one radial factor): only the A-bar reduction, all rows into dst1.
void emit_tri_helpers(Out& o, const Plan& p, bool stacked) {
  const int K2 = p.K, K = stacked ? p.K / 2 : p.K;
  if (stacked) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_tri_pack_phi(const real* __restrict__ p1, const real* __restrict__ p2, int e0, int e1,"
         " real* __restrict__ dst)");
  o.line(F("const i64 k = (i64)blockIdx.x * 256 + threadIdx.x, n = (i64)(e1 - e0) * %d;", K2));
  o.line("if (k >= n) return;");
  o.line(F("const i64 e = e0 + k / %d; const int q = (int)(k %% %d);", K2, K2));
  o.line(F("const real* src = q < %d ? p1 : p2;", K));
  o.line(F("dst[k] = src ? src[e * %d + (q %% %d)] : R(0);", K, K));
  o.close();
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_tri_pack_a(const real* __restrict__ a1, const real* __restrict__ a2, real* __restrict__ dst)");
  o.line(F("const i64 k = (i64)blockIdx.x * 256 + threadIdx.x, n = (i64)%d * %d;", K2, p.n_w));
  o.line("if (k >= n) return;");
  o.line(F("const i64 half = (i64)%d * %d;", K, p.n_w));
  o.line("const real* src = k < half ? a1 : a2;");
  o.line("dst[k] = src ? src[k < half ? k : k - half] : R(0);");
  o.close();
  }
  // A-bar of a receiver pass: the fixed-order sum of its nslot partial slots (as cgtp_a_reduce),
  // rows 0 .. K/2 - 1 added into dst1 and rows K/2 .. K - 1 into dst2 (each nullable).
  o.line("extern \"C\" __global__ void __launch_bounds__(512)");
  o.open("cgtp_tri_a_reduce(const real* __restrict__ ap, int nslot, real* __restrict__ dst1, real* __restrict__ dst2)");
  o.line(F("const int n = %d;", K2 * p.n_w));
  o.line("__shared__ real part[8][64];");
  o.line("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  o.line("const int k = (int)blockIdx.x * 64 + lane;");
  o.line("const int q = (nslot + 7) / 8, s0 = w * q, s1 = min(nslot, s0 + q);");
  o.line("real a0 = R(0), a1 = R(0), a2 = R(0), a3 = R(0);");
  o.open("if (k < n)");
  o.line("int s = s0;");
  o.line("for (; s + 3 < s1; s += 4) { a0 += ap[(i64)s * n + k]; a1 += ap[(i64)(s + 1) * n + k];"
         " a2 += ap[(i64)(s + 2) * n + k]; a3 += ap[(i64)(s + 3) * n + k]; }");
  o.line("for (; s < s1; ++s) a0 += ap[(i64)s * n + k];");
  o.close();
  o.line("part[w][lane] = (a0 + a1) + (a2 + a3);");
  o.line("__syncthreads();");
  o.open("if (w == 0 && k < n)");
  o.line("const real v = ((part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane])) +"
         " ((part[4][lane] + part[5][lane]) + (part[6][lane] + part[7][lane]));");
  o.line(F("const int half = %d;", K * p.n_w));
  if (stacked)
    o.line("if (k < half) { if (dst1) dst1[k] += v; } else { if (dst2) dst2[k - half] += v; }");
  else
    o.line("(void)half; (void)dst2; if (dst1) dst1[k] += v;");
  o.close();
  o.close();
}

// Zero-length edge check: per 256-edge block, the smallest sorted edge index whose vector
// pos[send] - pos[recv] + shift is exactly zero (INT_MAX if none), reduced in LDS in a fixed order.
void emit_check_edges(Out& o) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_check_edges(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, int n_edges, int* __restrict__ first)");
  o.line("__shared__ int sm[256];");
  o.line("const int tid = (int)threadIdx.x, e = (int)blockIdx.x * 256 + tid;");
  o.line("int bad = 0x7fffffff;");
  o.open("if (e < n_edges)");
  emit_edge_vector(o);
  o.line("if (rx * rx + ry * ry + rz * rz == R(0)) bad = e;");
  o.close();
  o.line("sm[tid] = bad;");
  o.line("__syncthreads();");
  o.open("for (int w = 128; w > 0; w >>= 1)");
  o.line("if (tid < w) sm[tid] = min(sm[tid], sm[tid + w]);");
  o.line("__syncthreads();");
  o.close();
  o.line("if (tid == 0) first[blockIdx.x] = sm[0];");
  o.close();
}

void emit_small_kernels(Out& o) {
  // Sum over the 64 lanes of a wave, the same value in every lane (fixed order).
  o.line("DEV real wave_total(real v) {");
  o.line("  v = rowsum(v);");
  o.line("  return (__shfl_rd(v, 0) + __shfl_rd(v, 16)) + (__shfl_rd(v, 32) + __shfl_rd(v, 48));");
  o.line("}");
  // pos-bar_i = sum over out-edges of e-bar - sum over in-edges of e-bar; one wave per node, lanes
  // stride the edge lists, then a fixed-order wave reduction.
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_pos_grad(const real* __restrict__ gev, const int* __restrict__ row_ptr,"
         " const int* __restrict__ src_ptr, const int* __restrict__ src_edge, int n, real* __restrict__ gpos)");
  o.line("const int i = (int)blockIdx.x, lane = (int)threadIdx.x;");
  o.line("if (i >= n) return;");
  o.line("real sx = R(0), sy = R(0), sz = R(0);");
  o.open("for (int k = src_ptr[i] + lane; k < src_ptr[i + 1]; k += 64)");
  o.line("const i64 e = src_edge[k];");
  o.line("sx += gev[3 * e]; sy += gev[3 * e + 1]; sz += gev[3 * e + 2];");
  o.close();
  o.open("for (int e = row_ptr[i] + lane; e < row_ptr[i + 1]; e += 64)");
  o.line("sx -= gev[3 * (i64)e]; sy -= gev[3 * (i64)e + 1]; sz -= gev[3 * (i64)e + 2];");
  o.close();
  o.line("sx = wave_total(sx); sy = wave_total(sy); sz = wave_total(sz);");
  o.line("if (lane == 0) { gpos[3 * (i64)i] = sx; gpos[3 * (i64)i + 1] = sy; gpos[3 * (i64)i + 2] = sz; }");
  o.close();
  // Source view of one receiver chunk: the out-edges of sender j whose sorted positions lie in
  // the chunk's range [e0, e1) form one run of j's ascending source-CSR list; beg[j], end[j]
  // bound that run (two binary searches, one thread per sender).
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open("cgtp_src_bounds(const int* __restrict__ src_ptr, const int* __restrict__ src_edge, int n, int e0, int e1,"
         " int* __restrict__ beg, int* __restrict__ end)");
  o.line("const int j = (int)blockIdx.x * 256 + (int)threadIdx.x;");
  o.line("if (j >= n) return;");
  o.line("int a = src_ptr[j], b = src_ptr[j + 1];");
  o.line("const int top = b;");
  o.line("while (a < b) { const int m = (a + b) >> 1; if (src_edge[m] < e0) a = m + 1; else b = m; }");
  o.line("beg[j] = a;");
  o.line("b = top;");
  o.line("while (a < b) { const int m = (a + b) >> 1; if (src_edge[m] < e1) a = m + 1; else b = m; }");
  o.line("end[j] = a;");
  o.close();
  // A-bar = sum over wave slots of the partials: block = 64 outputs x 8 slot ranges (one wave
  // each, four interleaved accumulators), combined in LDS in a fixed order.
  o.line("extern \"C\" __global__ void __launch_bounds__(512)");
  o.open("cgtp_a_reduce(const real* __restrict__ ap, int nslot, int n, real* __restrict__ gA)");
  o.line("__shared__ real part[8][64];");
  o.line("const int lane = (int)threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  o.line("const int k = (int)blockIdx.x * 64 + lane;");
  o.line("const int q = (nslot + 7) / 8, s0 = w * q, s1 = min(nslot, s0 + q);");
  o.line("real a0 = R(0), a1 = R(0), a2 = R(0), a3 = R(0);");
  o.open("if (k < n)");
  o.line("int s = s0;");
  o.line("for (; s + 3 < s1; s += 4) { a0 += ap[(i64)s * n + k]; a1 += ap[(i64)(s + 1) * n + k];"
         " a2 += ap[(i64)(s + 2) * n + k]; a3 += ap[(i64)(s + 3) * n + k]; }");
  o.line("for (; s < s1; ++s) a0 += ap[(i64)s * n + k];");
  o.close();
  o.line("part[w][lane] = (a0 + a1) + (a2 + a3);");
  o.line("__syncthreads();");
  o.line("if (w == 0 && k < n) gA[k] = ((part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane])) +"
         " ((part[4][lane] + part[5][lane]) + (part[6][lane] + part[7][lane]));");
  o.close();
}

}  // namespace gen

using namespace gen;

static std::vector<Task> make_forward_tasks(const Plan& p) {
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

static std::vector<Task> make_recv_backward_tasks(const Plan& p) {
  // Paths of every output block with the same multiplicity and 64-channel block are packed into
  // as few tasks as the register budget allows (first-fit, heaviest first): each task reduces its
  // per-edge partial sums over the channels once, however many output blocks it covers.  The
  // budget counts, per path, A and the A-bar accumulators (2K) plus the R table of folded paths.
  auto regs = [&](int pi) {
    const Path& P = p.paths[pi];
    return 2 * p.K + (folded(P) ? int(m12_pairs(P).size()) : 2 * P.l3 + 1);
  };
  std::map<std::pair<int, int>, std::vector<int>> by_key;  // (mul, channel block) -> paths
  for (int pi = 0; pi < int(p.paths.size()); ++pi) {
    const int mul = p.out[p.paths[pi].i_out].mul;
    for (int cb = 0; cb * 64 < mul; ++cb) by_key[{mul, cb}].push_back(pi);
  }
  std::vector<std::pair<int, Task>> tasks;  // (cost, task)
  for (auto& kv : by_key) {
    int budget = p.dtype == CGTP_F64 ? kRecvBudget / 2 : kRecvBudget;  // 64-bit values take two registers
    // Large paths read per lane take registers for their coefficient vectors; blocks whose rows
    // come by row broadcast (at most 32 channels in fp32) hold only a few chunks instead and take
    // twice the budget of those (l <= 6, 32 channels: 106 -> 68 tasks, 12.1 -> 11.7 ms; the full
    // budget drops to one wave per SIMD and measured 14.3 ms).
    if (p.vec_g) budget /= bcast_edges_per_wave(p, kv.first.first) > 1 ? kRecvLargeDiv / 2 : kRecvLargeDiv;
    std::vector<int> order = kv.second;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return regs(a) > regs(b); });
    std::vector<Task> bins;
    std::vector<int> used;
    for (int pi : order) {
      size_t b = 0;
      while (b < bins.size() && used[b] + regs(pi) > budget) ++b;
      if (b == bins.size()) {
        bins.push_back({p.paths[pi].i_out, kv.first.second, {}});
        used.push_back(0);
      }
      bins[b].paths.push_back(pi);
      used[b] += regs(pi);
    }
    for (Task& t : bins) {
      std::sort(t.paths.begin(), t.paths.end());
      int cost = 0;
      for (int pi : t.paths) cost += path_cost(p, p.paths[pi]);
      tasks.push_back({cost, t});
    }
  }
  std::stable_sort(tasks.begin(), tasks.end(), [](const auto& a, const auto& b) { return a.first > b.first; });
  std::vector<Task> t;
  for (auto& c : tasks) t.push_back(c.second);
  return t;
}

static std::vector<Task> make_dbl_recv_tasks(const Plan& p) {
  // Per path the receiver pass of the double backward holds A, its tangent and the A-bar tangent
  // accumulators (3K values per lane): one task per path up to K = 16 (two at K <= 8).  (Two per
  // task at K = 16 halve the per-edge channel reductions per path but drop to one wave per SIMD:
  // l <= 6, 32 channels, 27.2 -> 36.8 ms.)
  std::vector<Task> t;
  for (const Task& f : make_forward_tasks(p))
    for (const auto& S : a_subsets(p, f.paths, kRegBudget / 4)) t.push_back({f.group, f.cb, S});
  return t;
}

int bwd_row_stride(const Plan& p) { return (p.g_stride + p.sh_dim + 3) / 4 * 4; }

std::vector<int> recv_task_ycols(const Plan& p, const Task& T) {
  std::set<int> s;
  for (int pi : T.paths) {
    const Path& P = p.paths[pi];
    for (const CGTerm& t : P.terms) s.insert(P.l2 * P.l2 + t.m2);
  }
  return std::vector<int>(s.begin(), s.end());
}

int recv_task_width(const Plan& p, const Task& T) { return (p.K + int(recv_task_ycols(p, T).size()) + 3) / 4 * 4; }

int recv_partial_row(const Plan& p) { return task_tables(p).recv_row; }



static std::vector<Task> make_source_tasks(const Plan& p) {
  std::vector<Task> t;
  for (int k = 0; k < int(p.in.size()); ++k) {
    if (p.by_in[k].empty()) continue;
    int ncb = (p.in[k].mul + 63) / 64;
    for (int c = 0; c < ncb; ++c) t.push_back({k, c, p.by_in[k]});
  }
  return t;
}

// Task order of a launch, heaviest first (LunaTP section 4.2, "task ordering": path groups by
// their count of non-zero CG terms, descending, so that the last workgroups a launch dispatches
// are light ones).  A task's cost is the CG terms of its paths times its channels; tasks of one
// feature block (the channel blocks that share a workgroup) move together, ordered by the block's
// heaviest task; ties keep the plan order.
std::vector<Task> heaviest_first(const Plan& p, std::vector<Task> tasks) {
  auto cost = [&](const Task& t) {
    long long c = 0;
    for (int pi : t.paths) c += (long long)p.paths[pi].terms.size();
    return c * std::max(1, std::min(64, p.paths[t.paths[0]].n_w - 64 * t.cb));
  };
  std::map<int, long long> group_cost;
  for (const Task& t : tasks) group_cost[t.group] = std::max(group_cost[t.group], cost(t));
  std::stable_sort(tasks.begin(), tasks.end(), [&](const Task& a, const Task& b) {
    const long long ca = group_cost[a.group], cb = group_cost[b.group];
    if (ca != cb) return ca > cb;
    return a.group < b.group;
  });
  return tasks;
}

const TaskTables& task_tables(const Plan& p) {
  std::call_once(p.tables_once, [&p] {
    auto t = std::make_unique<TaskTables>();
    t->fwd = heaviest_first(p, make_forward_tasks(p));
    t->recv = make_recv_backward_tasks(p);
    std::stable_sort(t->recv.begin(), t->recv.end(), [&p](const Task& a, const Task& b) {
      auto c = [&p](const Task& t) {
        long long n = 0;
        for (int pi : t.paths) n += (long long)p.paths[pi].terms.size();
        return n;
      };
      return c(a) > c(b);
    });
    t->dbl_recv = make_dbl_recv_tasks(p);
    t->src = heaviest_first(p, make_source_tasks(p));
    for (const Task& k : t->recv) t->recv_row += recv_task_width(p, k);
    for (const Task& k : t->dbl_recv) t->dbl_row += dbl_task_width(p, k);
    p.tables = std::move(t);
  });
  return *p.tables;
}

TaskGroups task_groups(const std::vector<Task>& tasks) {
  TaskGroups g;
  std::vector<int> key;  // group of each entry of g.tasks
  for (int k = 0; k < int(tasks.size()); ++k) {
    auto it = std::find(key.begin(), key.end(), tasks[k].group);
    size_t at = it - key.begin();
    if (it == key.end()) {
      key.push_back(tasks[k].group);
      g.tasks.emplace_back();
    }
    auto& v = g.tasks[at];
    if (int(v.size()) <= tasks[k].cb) v.resize(tasks[k].cb + 1, -1);
    v[tasks[k].cb] = k;
    g.ncb = std::max(g.ncb, int(v.size()));
  }
  return g;
}

// Two waves split a receiver's edges in single precision; in double precision the latency of the
// (twice as many) coefficient loads is better hidden by more receivers in flight.
int fwd_split(const Plan& p) { return p.dtype == CGTP_F64 ? 1 : 2; }

const std::vector<Task>& forward_tasks(const Plan& p) { return task_tables(p).fwd; }
const std::vector<Task>& recv_backward_tasks(const Plan& p) { return task_tables(p).recv; }
const std::vector<Task>& dbl_recv_tasks(const Plan& p) { return task_tables(p).dbl_recv; }
const std::vector<Task>& source_tasks(const Plan& p) { return task_tables(p).src; }

int edge_partial_width(const Plan& p) { return (p.K + p.sh_dim + 3) / 4 * 4; }

// Feature layout conversion of one side (in / out) between ir_mul (block offset + m C + u) and
// mul_ir (block offset + u (2l+1) + m); one thread per element, reads or writes coalesced on the
// ir_mul side.
void emit_layout_kernel(Out& o, const std::vector<Block>& blocks, int width, const char* name) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open(std::string(name) + "(const real* __restrict__ src, real* __restrict__ dst, i64 total, int to_mul_ir)");
  o.line("const i64 k = (i64)blockIdx.x * 256 + threadIdx.x;");
  o.line("if (k >= total) return;");
  o.line(F("const i64 n = k / %d;", width));
  o.line(F("const int c = (int)(k - n * %d);", width));
  o.line("int off, mul, dim;");
  for (size_t b = 0; b < blocks.size(); ++b) {
    const Block& B = blocks[b];
    const std::string cond = b + 1 < blocks.size() ? F("if (c < %d) ", B.offset + B.size()) : std::string("");
    o.line((b ? "else " : "") + cond + F("{ off = %d; mul = %d; dim = %d; }", B.offset, B.mul, B.dim()));
  }
  o.line("const int r = c - off, m = r / mul, u = r - m * mul;");
  o.line(F("const i64 a = n * %d + c, t = n * %d + off + u * dim + m;", width, width));
  o.line("if (to_mul_ir) dst[t] = src[a]; else dst[a] = src[t];");
  o.close();
}

std::string generate_source(const Plan& p, const std::string& family, std::string* err) {
  Out o;
  if (family == "layout") {
    prelude(o, p, false, false);
    emit_layout_kernel(o, p.in, p.c_in, "cgtp_layout_in");
    emit_layout_kernel(o, p.out, p.c_out, "cgtp_layout_out");
    return o.s.str();
  }
  if (p.mode != CGTP_CHANNELWISE)
    return family == "uvw_rdbl" ? generate_uvw_radial_dbl_source(p, err) : generate_uvw_source(p, family, err);
  // fwdk: the conventional forward writing (and reading) the backward's row layout (G, then Y),
  // so that a backward called with the rows the forward kept needs no prep of its own.
  if (family == "fwd" || family == "fwds" || family == "fwdk") {
    const bool keep = family == "fwdk";
    prelude(o, p, false, false);
    emit_sh(o, p.lmax);
    emit_prep(o, p, keep);
    if (!keep) emit_check_edges(o);
    bool streamed = family == "fwds";
    auto tasks = forward_tasks(p);
    int nacc = 1;
    for (int k = 0; k < int(tasks.size()); ++k) {
      if (streamed) emit_fwd_streamed_task(o, p, k, tasks[k]);
      else emit_fwd_task(o, p, k, tasks[k], keep ? bwd_row_stride(p) : 0);
      int n = 0;
      for (int ob : out_blocks_of(p, tasks[k].paths)) n += p.out[ob].dim();
      nacc = std::max(nacc, n);
    }
    emit_node_dispatch(o, p, streamed ? "cgtp_fwd_streamed" : "cgtp_fwd", kFwdArgs, streamed ? "fwds_t" : "fwd_t",
                       task_groups(tasks), nacc);
    return o.s.str();
  }
  if (family == "dbl") return generate_dbl_source(p, err);
  if (family == "uvw_fwd" || family == "uvw_bwd") {
    *err = "fully connected families are generated by generate_uvw_source";
    return "";
  }
  // tri: the passes of the third-order derivative, generated for a plan with 2K radial values
  // (the parent plan's K twice): rows from an edge operand, the forward over the backward's row
  // layout, the receiver and source passes of the backward, edge finalisation without the
  // position chain, and the packing / accumulation helpers.
  // tri1: the same passes on the plan itself (K radial values), for terms with one weight factor.
  if (family == "tri" || family == "tri1") {
    const bool stacked = family == "tri";
    prelude(o, p, false, true);
    emit_prep_y(o, p);
    const std::vector<Task>& ft = forward_tasks(p);
    int nacc = 1;
    for (int k = 0; k < int(ft.size()); ++k) {
      emit_fwd_task(o, p, k, ft[k], bwd_row_stride(p), true);
      int n = 0;
      for (int ob : out_blocks_of(p, ft[k].paths)) n += p.out[ob].dim();
      nacc = std::max(nacc, n);
    }
    emit_node_dispatch(o, p, "cgtp_fwd", kFwdArgs, "fwd_t", task_groups(ft), nacc);
    auto rt = recv_backward_tasks(p);
    const int row = recv_partial_row(p);
    for (int k = 0, off = 0; k < int(rt.size()); off += recv_task_width(p, rt[k]), ++k)
      emit_bwd_recv_task(o, p, k, rt[k], off, row);
    emit_recv_dispatch(o, p, int(rt.size()));
    auto st = source_tasks(p);
    for (int k = 0; k < int(st.size()); ++k) emit_bwd_src_task(o, p, k, st[k]);
    emit_src_dispatch(o, p, int(st.size()));
    emit_recv_edge_final_y(o, p, rt, stacked);
    emit_small_kernels(o);
    emit_tri_helpers(o, p, stacked);
    return o.s.str();
  }
  if (family == "bwd") {
    prelude(o, p, true, true);
    emit_sh(o, p.lmax);
    emit_prep(o, p, true);
    auto rt = recv_backward_tasks(p);
    const int row = recv_partial_row(p);
    for (int k = 0, off = 0; k < int(rt.size()); off += recv_task_width(p, rt[k]), ++k)
      emit_bwd_recv_task(o, p, k, rt[k], off, row);
    emit_recv_dispatch(o, p, int(rt.size()));
    auto st = source_tasks(p);
    for (int k = 0; k < int(st.size()); ++k) emit_bwd_src_task(o, p, k, st[k]);
    emit_src_dispatch(o, p, int(st.size()));
    emit_recv_edge_final(o, p, rt);
    emit_small_kernels(o);
    return o.s.str();
  }
  *err = "unknown kernel family " + family;
  return "";
}

}  // namespace cgtp
