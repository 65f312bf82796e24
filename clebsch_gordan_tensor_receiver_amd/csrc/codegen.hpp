// Internal helpers shared by the kernel source generators (codegen.cpp: channelwise kernels and
// the shared edge/SH kernels; codegen_uvw.cpp: fully connected kernels).
#pragma once

#include <cstdarg>
#include <cstdio>
#include <functional>
#include <sstream>
#include <string>
#include <utility>
#include <vector>

#include "kernels.hpp"
#include "plan.hpp"

namespace cgtp {
namespace gen {

inline std::string F(const char* fmt, ...) {
  char buf[4096];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return buf;
}

inline std::string lit(double v) { return F("R(%.17g)", v); }

// Indented source text.
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

std::vector<std::vector<int>> subsets(const Plan& p, const std::vector<int>& paths);
// Consecutive subsets holding at most avail / K paths (A coefficients of K values per path).
std::vector<std::vector<int>> a_subsets(const Plan& p, const std::vector<int>& paths, int avail);
constexpr int kRegBudget = 64;  // registers per lane for A coefficients of one path subset

// Folded coefficients of large paths (more than kVecGPairs pairs) are read with 16-byte vector
// loads into VGPRs instead of scalar loads: `vz` is a per-lane zero the compiler cannot prove
// uniform (declared by emit_vz in every task of a plan with such paths).
inline bool path_vec(const Path& P) { return int(P.gpairs.size()) > kVecGPairs; }
void emit_vz(Out& o, const Plan& p);
// `vec` false: scalar loads whatever the path size (kernels where vector loads measured slower).
std::string gref(const Plan& p, int pi, int t, const std::string& row, const std::string& tag, bool vec = true);
// Coefficients of path pi referenced in increasing pair order t; a large path's row is read with
// 16-byte vector loads, other paths' values are scalar references.  `stream` false: the whole row
// is loaded up front.  `stream` true: it is read in chunks of kGvecChunk units, each loaded when
// the one before it is first used (at most two chunks live), with a scheduling barrier before
// each chunk that keeps the compiler from hoisting all of them to the top.
constexpr int kGvecChunk = 4;
class GStream {
 public:
  GStream(Out& o, const Plan& p, int pi, const std::string& row, const std::string& tag, bool stream);
  std::string ref(int t);

 private:
  void load(int chunk, bool barrier);
  Out& o_;
  const Plan& p_;
  int pi_, per_, n_, next_ = 0;
  bool vec_;
  std::string row_, tag_;
};
void prelude(Out& o, const Plan& p, bool dual, bool reduce);
// Radial values of the current edge (the phi input or the edge's G row), and the radial part of
// the edge-vector gradient (sr; needs rr = |r| and phi-bar registers <pb>0..K-1 in scope).
std::string phi_ptr(const Plan& p, const std::string& e, const std::string& grow);
void emit_radial_term(Out& o, const Plan& p, const std::string& pb);
void emit_sh(Out& o, int L);
void emit_edge_vector(Out& o);
void emit_prep(Out& o, const Plan& p, bool with_y = false);
std::vector<int> in_blocks_of(const Plan& p, const std::vector<int>& paths);
std::vector<int> out_blocks_of(const Plan& p, const std::vector<int>& paths);
void emit_recv_edge_loop(Out& o, const Plan& p, const std::vector<int>& blocks, const std::string& start,
                         const std::string& stride, const std::function<void()>& body, bool block_uc = false,
                         int row_stride = 0);
void emit_wave_combine(Out& o, const std::string& prefix, int n, int nw);
void emit_swaps(Out& o, const std::vector<std::pair<std::string, std::string>>& pairs, int width, bool f64);
void emit_edge_final(Out& o, const Plan& p, int ntask, int V);
void emit_recv_edge_final(Out& o, const Plan& p, const std::vector<Task>& tasks);
void emit_small_kernels(Out& o);
void emit_check_edges(Out& o);

}  // namespace gen

// Channelwise double backward (family "dbl").
std::string generate_dbl_source(const Plan& p, std::string* err);

// Fully connected (uvw) kernel families "uvw_fwd" and "uvw_bwd".
std::string generate_uvw_source(const Plan& p, const std::string& family, std::string* err);

}  // namespace cgtp
