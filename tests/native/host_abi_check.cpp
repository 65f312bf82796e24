// Host-side exercise of the library's C ABI for the address and undefined-behaviour sanitizers:
// plan construction for every standard irreps profile (paths, exact real CG tables), graph CSR
// construction on random and degenerate edge lists, workspace and state sizes for every operation,
// and the argument validation of the device entry points.  No GPU call is made.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "cgtp.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (%s)\n", what, cgtp_last_error());
    ++failures;
  }
}

struct Profile {
  const char *in, *sh, *out;
  cgtp_mode_t mode;
  cgtp_dtype_t dtype;
  int K;
};

}  // namespace

int main() {
  const Profile profiles[] = {
      {"8x0e+8x1o", "1x0e+1x1o+1x2e", "8x0e+8x1o+8x2e", CGTP_CHANNELWISE, CGTP_F64, 8},
      {"128x0e+128x1o+128x2e", "1x0e+1x1o+1x2e+1x3o", "128x0e+128x1o+128x2e+128x3o", CGTP_CHANNELWISE, CGTP_F32, 8},
      {"64x0e+64x1o+64x2e", "1x0e+1x1o+1x2e", "64x0e+64x1o+64x2e", CGTP_FULLY_CONNECTED, CGTP_F32, 8},
      {"32x0e+32x1o+32x2e+32x3o+32x4e+32x5o+32x6e", "1x0e+1x1o+1x2e+1x3o+1x4e+1x5o+1x6e",
       "32x0e+32x1o+32x2e+32x3o+32x4e+32x5o+32x6e", CGTP_CHANNELWISE, CGTP_F32, 16},
      {"128x0e+64x1e+32x2e", "1x0e+1x1e+1x2e", "128x0e+64x1e+32x2e", CGTP_CHANNELWISE, CGTP_F32, 8},
  };
  std::mt19937 rng(7);
  for (const Profile& pr : profiles) {
    cgtp_plan_t plan = nullptr;
    expect(cgtp_plan_create(pr.in, pr.sh, pr.out, pr.mode, pr.dtype, pr.K, &plan) == CGTP_OK, "plan_create");
    if (!plan) continue;
    cgtp_plan_info_t info;
    expect(cgtp_plan_info(plan, &info) == CGTP_OK, "plan_info");
    for (int k = 0; k < info.n_paths; ++k) {
      int32_t desc[9];
      expect(cgtp_plan_path(plan, k, desc) == CGTP_OK, "plan_path");
      int nnz = 0;
      expect(cgtp_plan_cg_table(plan, k, nullptr, nullptr, 0, &nnz) == CGTP_OK && nnz == desc[8], "cg_table count");
      const size_t nz = static_cast<size_t>(nnz);
      std::vector<int32_t> idx(3 * nz);
      std::vector<double> val(nz);
      expect(cgtp_plan_cg_table(plan, k, idx.data(), val.data(), nnz, &nnz) == CGTP_OK, "cg_table");
    }
    for (int n : {1, 2, 17, 300}) {
      std::uniform_int_distribution<int> node(0, n - 1);
      const int E = n == 1 ? 0 : 6 * n;
      const size_t ne = static_cast<size_t>(E);
      std::vector<int32_t> recv(ne), send(ne), image(3 * ne), perm(ne);
      for (int e = 0; e < E; ++e) {
        recv[e] = node(rng);
        send[e] = node(rng);
        for (int d = 0; d < 3; ++d) image[3 * size_t(e) + d] = int32_t(rng() % 3) - 1;
      }
      cgtp_graph_t g = nullptr;
      expect(cgtp_graph_build(n, E, recv.data(), send.data(), image.data(), perm.data(), &g) == CGTP_OK,
             "graph_build");
      if (!g) continue;
      const size_t nn = static_cast<size_t>(n);
      std::vector<int32_t> rp(nn + 1), col(ne + 1), sp(nn + 1), se(ne + 1);
      expect(cgtp_graph_export(g, rp.data(), col.data(), sp.data(), se.data()) == CGTP_OK, "graph_export");
      expect(cgtp_graph_set_order(g, 1) == CGTP_OK, "graph_set_order");
      for (int op = 0; op < 4; ++op) {
        size_t bytes = 0;
        cgtp_status_t st = cgtp_workspace_size(plan, g, cgtp_op_t(op), &bytes);
        const bool refused = pr.mode == CGTP_FULLY_CONNECTED && op == 3;
        expect(refused ? st == CGTP_ERR_UNSUPPORTED : (st == CGTP_OK && bytes >= 256), "workspace_size");
      }
      size_t sb = 0;
      cgtp_status_t st = cgtp_state_size(plan, g, &sb);
      expect(st == CGTP_OK || st == CGTP_ERR_UNSUPPORTED, "state_size");
      expect(cgtp_plan_set_scratch_budget(plan, 64 << 10) == CGTP_OK, "set_scratch_budget");
      for (int op = 0; op < 3; ++op) {
        size_t bytes = 0;
        expect(cgtp_workspace_size(plan, g, cgtp_op_t(op), &bytes) == CGTP_OK, "chunked workspace_size");
      }
      expect(cgtp_plan_set_scratch_budget(plan, size_t(256) << 20) == CGTP_OK, "restore budget");
      // Validation before any device work.
      expect(cgtp_conv_forward(plan, g, CGTP_CONVENTIONAL, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, 0, nullptr) == CGTP_ERR_INVALID_ARG, "forward null tensors");
      expect(cgtp_conv_triple_backward(plan, g, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                       nullptr, 0, nullptr) == CGTP_ERR_INVALID_ARG, "triple null tensors");
      expect(cgtp_graph_destroy(g) == CGTP_OK, "graph_destroy");
    }
    expect(cgtp_plan_destroy(plan) == CGTP_OK, "plan_destroy");
  }
  cgtp_plan_t bad = nullptr;
  expect(cgtp_plan_create("8x0e+bad", "1x0e", "8x0e", CGTP_CHANNELWISE, CGTP_F32, 8, &bad) == CGTP_ERR_INVALID_ARG,
         "malformed irreps");
  expect(cgtp_plan_create("8x7e", "1x0e", "8x7e", CGTP_CHANNELWISE, CGTP_F32, 8, &bad) == CGTP_ERR_UNSUPPORTED,
         "degree above 6");
  cgtp_graph_t g = nullptr;
  const int32_t r[1] = {5}, s[1] = {0};
  expect(cgtp_graph_build(3, 1, r, s, nullptr, nullptr, &g) == CGTP_ERR_INVALID_ARG, "node out of range");
  std::printf("host ABI check: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
