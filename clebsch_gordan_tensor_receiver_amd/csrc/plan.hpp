// Plan: irreps, paths, real Clebsch-Gordan tables and the work decomposition of the
// generated kernels.  Host-only C++17.
#pragma once

#include <cstddef>
#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "cgtp.h"

namespace cgtp {

constexpr int kMaxL = 6;

struct Block {
  int mul = 0, l = 0, parity = 1, offset = 0;
  int dim() const { return 2 * l + 1; }
  int size() const { return mul * dim(); }
};

struct CGTerm {
  int m1, m2, m3;
  double c;
};

// Structural pair (m1, m3) of a path with the CG terms that feed it:
// G[m1, m3] = sum_k c_k Y[m2_k]  (channel independent, one value per edge).
struct GPair {
  int m1, m3;
  std::vector<std::pair<int, double>> terms;  // (m2, c)
};

struct Path {
  int i_in, i_sh, i_out, l1, l2, l3;
  int w_off, n_w;
  int g_off;                      // first folded coefficient of this path in a G row
  std::vector<CGTerm> terms;      // non-zero real CG entries, row-major
  std::vector<GPair> gpairs;      // ordered by m3, then m1
};

// Kernel family state (compiled code objects and loaded modules per device).
struct KernelSet;
struct TaskTables;

// Paths with more (m1, m3) pairs than this read their folded coefficients through vector loads
// (the scalar register file cannot hold them per edge).
constexpr int kVecGPairs = 48;

struct Plan {
  std::vector<Block> in, sh, out;
  std::vector<Path> paths;
  cgtp_mode_t mode;
  cgtp_dtype_t dtype;
  int K = 0;
  int c_in = 0, c_out = 0, sh_dim = 0, lmax = 0, n_w = 0;
  int g_width = 0;     // folded coefficients per edge (sum over paths of gpairs, with alignment)
  bool vec_g = false;  // some path has more than kVecGPairs pairs: path blocks are 4-aligned
  int g_stride = 0;    // padded row stride of G in elements
  int cg_nnz = 0;
  size_t scratch_budget = size_t(256) << 20;
  // Radial basis computed from |r| inside the kernels (cgtp_plan_set_radial): 0 = none (phi is an
  // input), 1 = Bessel with the p = 6 polynomial envelope, 2 = Gaussian.  The K values of an edge
  // sit in its G row at phi_off.
  int radial = 0;
  double r_cut = 0.0;
  int phi_off = 0;
  // Paths into each output block / out of each input block, in path order.
  std::vector<std::vector<int>> by_out, by_in;
  std::string key;     // canonical description used to name and cache kernels
  std::string irreps_in_s, irreps_sh_s, irreps_out_s;  // as given to build_plan
  // The same irreps with 2K radial values, whose kernels run the third-order passes (a weight
  // phi_1 A_1 + phi_2 A_2 as one product of stacked factors); built on first use, under `mu`.
  std::unique_ptr<Plan> tri;
  // The same irreps and K without a radial basis: the fully connected double backward of a plan
  // with one runs on it with phi and phi-dot materialised per edge; built on first use, under `mu`.
  std::unique_ptr<Plan> plain;
  std::unique_ptr<KernelSet> kernels;
  std::mutex mu;
  mutable std::once_flag tables_once;              // task lists (kernels.hpp), built on first use
  mutable std::unique_ptr<TaskTables> tables;
  size_t elem() const { return dtype == CGTP_F64 ? 8 : 4; }
  ~Plan();
};

// Parse "8x0e+8x1o" into blocks; returns false with a message on error.
bool parse_irreps(const std::string& s, std::vector<Block>* out, std::string* err);

// Complex Clebsch-Gordan <l1 m1 l2 m2 | l3 m3> (Racah sum in long double).
long double complex_cg(int l1, int m1, int l2, int m2, int l3, int m3);

// Real CG tensor (2l1+1)(2l2+1)(2l3+1), row-major, with the documented basis and sign rule.
std::vector<double> real_cg(int l1, int l2, int l3);

cgtp_status_t build_plan(const char* irreps_in, const char* irreps_sh, const char* irreps_out,
                         cgtp_mode_t mode, cgtp_dtype_t dtype, int K, Plan* p, std::string* err);

}  // namespace cgtp
