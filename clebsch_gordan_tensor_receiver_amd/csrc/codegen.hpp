// Internal helpers shared by the kernel source generators (codegen.cpp: channelwise kernels and
// the shared edge/SH kernels; codegen_uvw.cpp: fully connected kernels).
#pragma once

#include <array>
#include <cstdarg>
#include <cstdio>
#include <functional>
#include <sstream>
#include <set>
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
// Coefficient rows read by row broadcast (fp32, one edge per 16-lane row, `r16_` = lane & 15 in
// scope): the 64-value chunks of row pointer `row` loaded so far (gchunk, one 16-byte load per
// lane), named gc<tag><chunk>; `lim` is the row length in values.  `order` lists the chunks in
// the order the body first uses them (chunks_of): when a chunk is first used, the next
// kChunkAhead chunks of the list are loaded too, ahead of a scheduling barrier, so that their
// latency overlaps the arithmetic on the chunks before them.
constexpr int kChunkAhead = 2;
struct RowChunks {
  int lim;
  std::string row = "g", tag = "";
  std::vector<int> order = {};
  std::set<int> loaded = {};
  std::set<int> used = {};
};
// Chunks (64 values) touched by the value ranges [first, second) of a row, in order of first use.
std::vector<int> chunks_of(const std::vector<std::pair<int, int>>& ranges);
// Value ranges of the coefficient rows of the given paths, in path order.
std::vector<std::pair<int, int>> g_ranges(const Plan& p, const std::vector<int>& paths);
// Statement `dst = G[idx] * xop` (first) or `dst += G[idx] * xop`, G[idx] read from its chunk by
// row broadcast; the chunk (and the kChunkAhead after it) is loaded on its first use.
std::string bcast_term(Out& o, RowChunks& rc, int idx, const std::string& dst, const std::string& xop, bool first);
// Edges per wave step of the channelwise passes that read coefficient rows per edge.
int bcast_edges_per_wave(const Plan& p, int mul);
void prelude(Out& o, const Plan& p, bool dual, bool reduce);
// Radial values of the current edge (the phi input or the edge's G row), and the radial part of
// the edge-vector gradient (sr; needs rr = |r| and phi-bar registers <pb>0..K-1 in scope).
std::string phi_ptr(const Plan& p, const std::string& e, const std::string& grow);
void emit_radial_term(Out& o, const Plan& p, const std::string& pb);
void emit_sh(Out& o, int L);
void emit_edge_vector(Out& o);
void emit_prep(Out& o, const Plan& p, bool with_y = false);
// LDS-staged 16-byte stores of per-edge rows (lane = edge); see codegen.cpp.
void emit_staged_rows(Out& o, const Plan& p, std::vector<std::string> vals, int stride);
std::vector<int> in_blocks_of(const Plan& p, const std::vector<int>& paths);
std::vector<int> out_blocks_of(const Plan& p, const std::vector<int>& paths);
// nE > 1 (2 or 4): the wave's lanes form nE groups of 64 / nE channels and take nE consecutive
// edges of its share at a time, group h the h-th (blocks of at most 64 / nE channels); the edge
// index e, sender j, row pointer g and phi values f<q> are then per lane (zero phi for a group
// past the last edge).
void emit_recv_edge_loop(Out& o, const Plan& p, const std::vector<int>& blocks, const std::string& start,
                         const std::string& stride, const std::function<void()>& body, bool block_uc = false,
                         int row_stride = 0, int nE = 1);
void emit_wave_combine(Out& o, const std::string& prefix, int n, int nw);
void emit_swaps(Out& o, const std::vector<std::pair<std::string, std::string>>& pairs, int width, bool f64);
// Per-edge partial columns v0..v(V-1) of a wave whose lane groups of gsz lanes (16 or 32) each hold
// one edge (`lane`, `ok_` in scope; V even): summed over each group's lanes and stored, column k
// at dst[64 k] for an edge that is valid, dst = `dst_expr` evaluated per lane.  Only the first
// nreal columns are read later; with 16-lane groups the rest (padding) are not summed in fp32.
void emit_group_reduce_store(Out& o, int V, int nreal, int gsz, bool f64, const std::string& dst_expr);
// Sums over the 16 lanes of each row of the fp32 registers v0..v(n-1) (row r of register k holds
// the partials of one output) by an in-row transposition, and the statements `store(kk, val)`
// that store them (see codegen.cpp).
void emit_row_reduce_store(Out& o, int n, const std::string& ok,
                           const std::function<std::string(const std::string&, const std::string&)>& store);
void emit_edge_final(Out& o, const Plan& p, int ntask, int V);
void emit_recv_edge_final(Out& o, const Plan& p, const std::vector<Task>& tasks);
void emit_small_kernels(Out& o);
// Gdot-row preps and the edge finalisation of the fully connected double backward (ntask edge
// tasks of V partial columns each).
void emit_uvw_dbl_kernels(Out& o, const Plan& p, int ntask, int V);
void emit_check_edges(Out& o);

}  // namespace gen

// Channelwise double backward (family "dbl").
std::string generate_dbl_source(const Plan& p, std::string* err);
// Fully connected double backward with an in-kernel radial basis (family "uvw_rdbl"): phi and its
// tangent per edge, and the radial terms of the edge-vector gradient.
std::string generate_uvw_radial_dbl_source(const Plan& p, std::string* err);

// Fully connected (uvw) kernel families "uvw_fwd" and "uvw_bwd".
std::string generate_uvw_source(const Plan& p, const std::string& family, std::string* err);

}  // namespace cgtp
