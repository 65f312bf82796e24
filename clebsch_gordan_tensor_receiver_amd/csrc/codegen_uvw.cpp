// Fully connected (uvw) kernels: the streamed schedule of Sobek section 4.2-4.3.
//
// Forward (Eqs. 32-35), per output block g:
//   uvw_state (lane = input channel u): S_i[(m3)][(pi, q, u)] = sum_j phi_ij,q C_pi,u,m3(x_j, Y_ij),
//       accumulated in registers over the receiver's edges, written as rows of a receiver-chunk
//       matrix S_g (rows (i, m3), columns (pi, q, u));
//   gemm_fwd_g (MFMA): m_g = S_g A_g with A_g[(pi, q, u)][w] = A[q, w_off_pi + u C_out + w].
// Backward (Eq. 36 and its edge/source parts), per receiver chunk:
//   uvw_state again (S), gemm_sbar_g: Sbar_g = mbar_g A_g^T, gemm_abar_g: A-bar_g += S_g^T mbar_g
//   (split over rows, partials summed in a fixed order);
//   uvw_edge (lane = u): per edge phi-bar_q = sum Sbar[q] C and Y-bar from
//   Cbar[m3] = sum_q phi_q Sbar[q][m3], reduced over channels; edge_final and pos_grad as in the
//   channelwise path.
// and per sender chunk (x-bar without edge-sized buffers): the source-side state
//   Z_j[(m1)][(pi, q, w)] = sum_{e: j -> i} phi_e,q sum_m3 G_e[m1, m3] mbar_i[m3][w]
//   (uvw_zstate, lane = output channel w, over the source CSR), then gemm_xbar_b:
//   x-bar_j[m1][u] = sum_{(pi, q, w)} Z_j[m1][(pi, q, w)] A[q, w_off_pi + u C_out + w].
#include <algorithm>
#include <functional>
#include <set>

#include "codegen.hpp"

namespace cgtp {

using namespace gen;

namespace {

constexpr int kStateBudget = 96;   // receiver/source state registers per lane per task

struct Side {                 // one output block (receiver side) or input block (source side)
  int blk;                    // block index
  std::vector<int> paths;
  int d;                      // 2l + 1 of the block
  int mul;                    // channels of the block
  std::vector<int> col_off;   // per path: first column of the path in a state row
  std::vector<int> cmul;      // per path: channels along the state columns (mul_in or mul_out)
  int D = 0, ld = 0;          // columns and padded row stride
};

std::vector<Side> recv_sides(const Plan& p) {
  std::vector<Side> v;
  for (int k = 0; k < int(p.out.size()); ++k) {
    if (p.by_out[k].empty()) continue;
    Side s{k, p.by_out[k], p.out[k].dim(), p.out[k].mul, {}, {}};
    for (int pi : s.paths) {
      s.col_off.push_back(s.D);
      s.cmul.push_back(p.in[p.paths[pi].i_in].mul);
      s.D += p.K * p.in[p.paths[pi].i_in].mul;
    }
    s.ld = (s.D + 3) / 4 * 4;
    v.push_back(s);
  }
  return v;
}

std::vector<Side> send_sides(const Plan& p) {
  std::vector<Side> v;
  for (int k = 0; k < int(p.in.size()); ++k) {
    if (p.by_in[k].empty()) continue;
    Side s{k, p.by_in[k], p.in[k].dim(), p.in[k].mul, {}, {}};
    for (int pi : s.paths) {
      s.col_off.push_back(s.D);
      s.cmul.push_back(p.out[p.paths[pi].i_out].mul);
      s.D += p.K * p.out[p.paths[pi].i_out].mul;
    }
    s.ld = (s.D + 3) / 4 * 4;
    v.push_back(s);
  }
  return v;
}

struct StateTask {
  int side;                  // index into recv_sides / send_sides
  std::vector<int> idx;      // indices into side.paths
  int cb;
};

std::vector<StateTask> state_tasks(const Plan& p, const std::vector<Side>& sides, int budget_per_path_fn(const Plan&, const Side&, int)) {
  std::vector<StateTask> t;
  for (int s = 0; s < int(sides.size()); ++s) {
    const Side& S = sides[s];
    std::vector<std::vector<int>> groups;
    int used = 0;
    for (int k = 0; k < int(S.paths.size()); ++k) {
      int cost = budget_per_path_fn(p, S, k);
      if (groups.empty() || used + cost > kStateBudget) {
        groups.push_back({});
        used = 0;
      }
      groups.back().push_back(k);
      used += cost;
    }
    for (auto& g : groups) {
      int mmax = 0;
      for (int k : g) mmax = std::max(mmax, S.cmul[k]);
      for (int cb = 0; cb < (mmax + 63) / 64; ++cb) t.push_back({s, g, cb});
    }
  }
  return t;
}

int recv_state_cost(const Plan& p, const Side& S, int) { return p.K * S.d; }
int send_state_cost(const Plan& p, const Side& S, int) { return p.K * S.d; }

// Row offset in A of column c of a receiver-side state (pi, q, u): q N_w + w_off + u C_out.
void emit_brow(Out& o, const Plan& p, const Side& S, const std::string& name) {
  o.open("DEV i64 " + name + "(int c)");
  for (size_t k = 0; k < S.paths.size(); ++k) {
    const Path& P = p.paths[S.paths[k]];
    const int mul_in = S.cmul[k], mul_out = p.out[P.i_out].mul;
    const int hi = S.col_off[k] + p.K * mul_in;
    o.line(F("if (c < %d) { const int r = c - %d, q = r / %d, u = r - q * %d;"
             " return (i64)q * %d + %d + (i64)u * %d; }",
             hi, S.col_off[k], mul_in, mul_in, p.n_w, P.w_off, mul_out));
  }
  o.line("return 0;");
  o.close();
}

// Row base and channel stride in A of column c of a source-side state (pi, q, w):
// A[q, w_off + u C_out + w] = base + u * stride.
void emit_bz(Out& o, const Plan& p, const Side& S, const std::string& name) {
  o.open("DEV i64 " + name + "(int c, int& stride)");
  for (size_t k = 0; k < S.paths.size(); ++k) {
    const Path& P = p.paths[S.paths[k]];
    const int mul_out = S.cmul[k];
    const int hi = S.col_off[k] + p.K * mul_out;
    o.line(F("if (c < %d) { const int r = c - %d, q = r / %d, w = r - q * %d; stride = %d;"
             " return (i64)q * %d + %d + w; }",
             hi, S.col_off[k], mul_out, mul_out, mul_out, p.n_w, P.w_off));
  }
  o.line("stride = 0; return 0;");
  o.close();
}

struct GemmSpec {
  std::string name, args, a_at, b_at, store;
  int N;
  bool a_kfast, b_kfast, split;
  // 16-byte tile loads: a_at / b_at are element lvalues contiguous along their fast index whose
  // 4-aligned groups are 16-byte aligned when the base pointers a_ptr and b_ptr are (every
  // multiplicity a multiple of 4); checked at run time, else one element per load.
  bool vec = false;
  std::string a_ptr, b_ptr;
};

// Every feature block's multiplicity is a multiple of 4: all row strides, block offsets and
// weight offsets are then multiples of 4 elements.
bool gemm_vec_ok(const Plan& p) {
  for (auto& b : p.in)
    if (b.mul % 4) return false;
  for (auto& b : p.out)
    if (b.mul % 4) return false;
  return true;
}

// LDS-tiled MFMA GEMM: 64 x 64 output tile per 4-wave workgroup, K staged 32 at a time, each wave
// a 32 x 32 quarter as 2 x 2 MFMA 16x16x4 tiles.  A K-fast B operand (stored 32 k values of one
// column by 32 lanes) has its tile columns XOR-swizzled inside aligned groups of 16 by
// (k / 2) mod 16: the stores then hit 32 distinct banks instead of 2, the MFMA reads stay
// conflict-free.  C[r][c] = sum_k A(r, k) B(k, c) over
// k in [kb, ke); `store` writes value v at (r, c).  Two LDS buffers: the next K slice is loaded
// into registers while the current one feeds the MFMAs, then stored to the other buffer, so one
// barrier per slice suffices and the global loads overlap the matrix work.
void emit_gemm(Out& o, const GemmSpec& g) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open(g.name + "(" + g.args + ", int M, int Kd, int kper)");
  o.line("__shared__ real As[2][64 * 34];");
  o.line("__shared__ real Bs[2][32 * 80];");
  o.line("const int tid = (int)threadIdx.x, lane = tid & 63, wv = tid >> 6;");
  o.line("const int r0 = (int)blockIdx.x * 64, c0 = (int)blockIdx.y * 64;");
  if (g.split) {
    o.line("const int kb = (int)blockIdx.z * kper, ke = min(Kd, kb + kper);");
  } else {
    o.line("const int kb = 0, ke = Kd; (void)kper;");
  }
  o.line("acc4 a00 = {0, 0, 0, 0}, a01 = {0, 0, 0, 0}, a10 = {0, 0, 0, 0}, a11 = {0, 0, 0, 0};");
  o.line("real ra[8], rb[8];");
  // 16-byte loads only where the B operand's columns are the fast index: K-fast B groups would
  // store four k rows of one column to LDS at once and collide in its banks (measured slower,
  // also with only the A operand vectorized).
  const bool vec = g.vec && !g.b_kfast;
  if (vec)
    o.line("const bool vec_ = ((unsigned long long)" + g.a_ptr + " & 15) == 0 && ((unsigned long long)" + g.b_ptr +
           " & 15) == 0;");
  // Both operands' vector forms under one vec_ branch, else their element forms.
  auto twoway = [&](const std::function<void()>& vf, const std::function<void()>& sf) {
    if (vec) {
      o.open("if (vec_)");
      vf();
      o.close();
      o.open("else");
      sf();
      o.close();
    } else {
      o.open("");
      sf();
      o.close();
    }
  };
  // Vector form: per operand 512 groups of 4 elements along the fast index, 2 per thread; a
  // group that leaves the matrix is read element by element.
  auto vgroup = [&](const std::string& dst, const std::string& at, const std::string& full,
                    const std::string& elem_var, const std::string& elem_val, const std::string& cond) {
    o.open("if (" + full + ")");
    o.line("const Q4 q_ = *(const Q4*)&(" + at + ");");
    o.line(dst + "[4 * t] = q_.a; " + dst + "[4 * t + 1] = q_.b; " + dst + "[4 * t + 2] = q_.c; " + dst +
           "[4 * t + 3] = q_.d;");
    o.close();
    o.open("else");
    o.open("for (int i = 0; i < 4; ++i)");
    o.line("const int " + elem_var + " = " + elem_val + ";");
    o.line(dst + "[4 * t + i] = (" + cond + ") ? (" + at + ") : R(0);");
    o.close();
    o.close();
  };
  auto vloadA = [&]() {
    o.open("for (int t = 0; t < 2; ++t)");
    o.line("const int v = t * 256 + tid;");
    if (g.a_kfast) {
      o.line("const int r = r0 + (v >> 3), kq = (v & 7) << 2, k = k0_ + kq;");
      vgroup("ra", g.a_at, "r < M && k + 3 < ke", "k", "k0_ + kq + i", "r < M && k < ke");
    } else {
      o.line("const int rq = (v & 15) << 2, r = r0 + rq, k = k0_ + (v >> 4);");
      vgroup("ra", g.a_at, "r + 3 < M && k < ke", "r", "r0 + rq + i", "r < M && k < ke");
    }
    o.close();
  };
  auto vloadB = [&]() {
    o.open("for (int t = 0; t < 2; ++t)");
    o.line("const int v = t * 256 + tid;");
    o.line("const int cq = (v & 15) << 2, c = c0 + cq, k = k0_ + (v >> 4);");
    vgroup("rb", g.b_at, F("k < ke && c + 3 < %d", g.N), "c", "c0 + cq + i", F("k < ke && c < %d", g.N));
    o.close();
  };
  auto sload = [&]() {
    o.open("for (int t = 0; t < 8; ++t)");
    o.line("const int id = t * 256 + tid;");
    o.line(g.a_kfast ? "const int rr = id >> 5, kk = id & 31;" : "const int rr = id & 63, kk = id >> 6;");
    o.line("const int r = r0 + rr, k = k0_ + kk;");
    o.line("ra[t] = (r < M && k < ke) ? (" + g.a_at + ") : R(0);");
    o.close();
    o.open("for (int t = 0; t < 8; ++t)");
    o.line("const int id = t * 256 + tid;");
    o.line(g.b_kfast ? "const int cc = id >> 5, kk = id & 31;" : "const int cc = id & 63, kk = id >> 6;");
    o.line("const int c = c0 + cc, k = k0_ + kk;");
    o.line(F("rb[t] = (k < ke && c < %d) ? (", g.N) + g.b_at + ") : R(0);");
    o.close();
  };
  // Global -> registers for the K slice starting at k0.
  auto load = [&](const std::string& k0) {
    o.open("");
    o.line("const int k0_ = " + k0 + ";");
    twoway([&] { vloadA(); vloadB(); }, sload);
    o.close();
  };
  // Registers -> LDS buffer `buf`.
  auto store = [&](const std::string& buf) {
    twoway([&] {
      o.open("for (int t = 0; t < 2; ++t)");
      o.line("const int v = t * 256 + tid;");
      o.open("");
      if (g.a_kfast) {
        o.line("const int rr = v >> 3, kq = (v & 7) << 2;");
        o.line("for (int i = 0; i < 4; ++i) As[" + buf + "][rr * 34 + kq + i] = ra[4 * t + i];");
      } else {
        o.line("const int rq = (v & 15) << 2, kk = v >> 4;");
        o.line("for (int i = 0; i < 4; ++i) As[" + buf + "][(rq + i) * 34 + kk] = ra[4 * t + i];");
      }
      o.close();
      o.line("const int cq = (v & 15) << 2, kk = v >> 4;");
      o.line("for (int i = 0; i < 4; ++i) Bs[" + buf + "][kk * 80 + cq + i] = rb[4 * t + i];");
      o.close();
    }, [&] {
      o.open("for (int t = 0; t < 8; ++t)");
      o.line("const int id = t * 256 + tid;");
      o.line(g.a_kfast ? "const int rr = id >> 5, kk = id & 31;" : "const int rr = id & 63, kk = id >> 6;");
      o.line("As[" + buf + "][rr * 34 + kk] = ra[t];");
      o.close();
      o.open("for (int t = 0; t < 8; ++t)");
      o.line("const int id = t * 256 + tid;");
      o.line(g.b_kfast ? "const int cc = id >> 5, kk = id & 31;" : "const int cc = id & 63, kk = id >> 6;");
      o.line(g.b_kfast ? "Bs[" + buf + "][kk * 80 + (cc ^ ((kk >> 1) & 15))] = rb[t];"
                       : "Bs[" + buf + "][kk * 80 + cc] = rb[t];");
      o.close();
    });
  };
  o.open("if (kb < ke)");
  load("kb");
  store("0");
  o.close();
  o.line("__syncthreads();");
  o.open("for (int k0 = kb, cur = 0; k0 < ke; k0 += 32, cur ^= 1)");
  o.line("const bool more = k0 + 32 < ke;");
  o.open("if (more)");
  load("k0 + 32");
  o.close();
  o.open("for (int s = 0; s < 8; ++s)");
  o.line("const int ka = s * 4 + (lane >> 4);");
  o.line("const real x0 = As[cur][(32 * (wv >> 1) + (lane & 15)) * 34 + ka];");
  o.line("const real x1 = As[cur][(32 * (wv >> 1) + 16 + (lane & 15)) * 34 + ka];");
  o.line(g.b_kfast ? "const int sw = (ka >> 1) & 15;" : "const int sw = 0;");
  o.line("const real y0 = Bs[cur][ka * 80 + ((32 * (wv & 1) + (lane & 15)) ^ sw)];");
  o.line("const real y1 = Bs[cur][ka * 80 + ((32 * (wv & 1) + 16 + (lane & 15)) ^ sw)];");
  o.line("a00 = MFMA(x0, y0, a00); a01 = MFMA(x0, y1, a01); a10 = MFMA(x1, y0, a10); a11 = MFMA(x1, y1, a11);");
  o.close();
  o.open("if (more)");
  store("cur ^ 1");
  o.close();
  o.line("__syncthreads();");
  o.close();
  o.open("for (int q = 0; q < 4; ++q)");
  o.line("const int wr = q >> 1, wc = q & 1;");
  o.line("const acc4 acc = q == 0 ? a00 : (q == 1 ? a01 : (q == 2 ? a10 : a11));");
  o.open("for (int rr = 0; rr < 4; ++rr)");
  // Accumulator layout: lane l, element rr holds row 4 (l / 16) + rr (f32) or 4 rr + l / 16 (f64).
  o.line("const int r = r0 + 32 * (wv >> 1) + 16 * wr + ROWOF(lane, rr);");
  o.line("const int c = c0 + 32 * (wv & 1) + 16 * wc + (lane & 15);");
  o.line(F("if (r < M && c < %d) { const real v = acc[rr]; ", g.N) + g.store + " }");
  o.close();
  o.close();
  o.close();
}

// GEMM of depth at most 64 (no K split): the 64 x Kd panel of A is loaded into LDS once and the
// workgroup sweeps kSbarPanelTiles column tiles of 64, loading the next B tile into registers
// while the current one feeds the MFMAs (same tile layout, swizzle and wave quarters as
// emit_gemm; element loads).
void emit_gemm_panel(Out& o, const GemmSpec& g) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open(g.name + "(" + g.args + ", int M, int Kd, int kper)");
  o.line("__shared__ real As[2][64 * 34];");
  o.line("__shared__ real Bs[2][32 * 80];");
  o.line("const int tid = (int)threadIdx.x, lane = tid & 63, wv = tid >> 6;");
  o.line("const int r0 = (int)blockIdx.x * 64, ke = Kd;");
  o.line("(void)kper;");
  o.line("real rb0[8], rb1[8];");
  for (int sl = 0; sl < 2; ++sl) {
    o.open("for (int t = 0; t < 8; ++t)");
    o.line("const int id = t * 256 + tid;");
    o.line(g.a_kfast ? "const int rr = id >> 5, kk = id & 31;" : "const int rr = id & 63, kk = id >> 6;");
    o.line(F("const int r = r0 + rr, k = %d + kk;", 32 * sl));
    o.line(F("As[%d][rr * 34 + kk] = (r < M && k < ke) ? (", sl) + g.a_at + ") : R(0);");
    o.close();
  }
  auto loadB = [&](const std::string& c0) {
    o.open("");
    o.line("const int cb_ = " + c0 + ";");
    for (int sl = 0; sl < 2; ++sl) {
      o.open("for (int t = 0; t < 8; ++t)");
      o.line("const int id = t * 256 + tid;");
      o.line(g.b_kfast ? "const int cc = id >> 5, kk = id & 31;" : "const int cc = id & 63, kk = id >> 6;");
      o.line(F("const int c = cb_ + cc, k = %d + kk;", 32 * sl));
      o.line(F("rb%d[t] = (k < ke && c < %d) ? (", sl, g.N) + g.b_at + ") : R(0);");
      o.close();
    }
    o.close();
  };
  auto storeB = [&] {
    for (int sl = 0; sl < 2; ++sl) {
      o.open("for (int t = 0; t < 8; ++t)");
      o.line("const int id = t * 256 + tid;");
      o.line(g.b_kfast ? "const int cc = id >> 5, kk = id & 31;" : "const int cc = id & 63, kk = id >> 6;");
      o.line(g.b_kfast ? F("Bs[%d][kk * 80 + (cc ^ ((kk >> 1) & 15))] = rb%d[t];", sl, sl)
                       : F("Bs[%d][kk * 80 + cc] = rb%d[t];", sl, sl));
      o.close();
    }
  };
  o.line(F("const int ct0 = (int)blockIdx.y * %d;", kSbarPanelTiles));
  loadB("ct0 * 64");
  storeB();
  o.line("__syncthreads();");
  o.open(F("for (int ct = 0; ct < %d; ++ct)", kSbarPanelTiles));
  o.line("const int c0 = (ct0 + ct) * 64;");
  o.line(F("if (c0 >= %d) break;", g.N));
  o.line(F("const bool more = ct + 1 < %d && c0 + 64 < %d;", kSbarPanelTiles, g.N));
  o.open("if (more)");
  loadB("c0 + 64");
  o.close();
  o.line("acc4 a00 = {0, 0, 0, 0}, a01 = {0, 0, 0, 0}, a10 = {0, 0, 0, 0}, a11 = {0, 0, 0, 0};");
  o.open("for (int s = 0; s < 16; ++s)");
  o.line("const int cur = s >> 3, ka = (s & 7) * 4 + (lane >> 4);");
  o.line("const real x0 = As[cur][(32 * (wv >> 1) + (lane & 15)) * 34 + ka];");
  o.line("const real x1 = As[cur][(32 * (wv >> 1) + 16 + (lane & 15)) * 34 + ka];");
  o.line(g.b_kfast ? "const int sw = (ka >> 1) & 15;" : "const int sw = 0;");
  o.line("const real y0 = Bs[cur][ka * 80 + ((32 * (wv & 1) + (lane & 15)) ^ sw)];");
  o.line("const real y1 = Bs[cur][ka * 80 + ((32 * (wv & 1) + 16 + (lane & 15)) ^ sw)];");
  o.line("a00 = MFMA(x0, y0, a00); a01 = MFMA(x0, y1, a01); a10 = MFMA(x1, y0, a10); a11 = MFMA(x1, y1, a11);");
  o.close();
  o.open("for (int q = 0; q < 4; ++q)");
  o.line("const int wr = q >> 1, wc = q & 1;");
  o.line("const acc4 acc = q == 0 ? a00 : (q == 1 ? a01 : (q == 2 ? a10 : a11));");
  o.open("for (int rr = 0; rr < 4; ++rr)");
  o.line("const int r = r0 + 32 * (wv >> 1) + 16 * wr + ROWOF(lane, rr);");
  o.line("const int c = c0 + 32 * (wv & 1) + 16 * wc + (lane & 15);");
  o.line(F("if (r < M && c < %d) { const real v = acc[rr]; ", g.N) + g.store + " }");
  o.close();
  o.close();
  o.line("__syncthreads();");
  o.open("if (more)");
  storeB();
  o.line("__syncthreads();");
  o.close();
  o.close();
  o.close();
}

// Fixed-order sum of the split-K partials of a GEMM (part[z][r][c], z < nsplit) and the GEMM's
// scatter store of the result.
void emit_gemm_reduce(Out& o, const GemmSpec& g, const std::string& args) {
  o.line("extern \"C\" __global__ void __launch_bounds__(256)");
  o.open(g.name + "_reduce(const real* __restrict__ part, int nsplit, int M, " + args + ")");
  o.line("const i64 id = (i64)blockIdx.x * 256 + threadIdx.x;");
  o.line(F("const i64 MN = (i64)M * %d;", g.N));
  o.line("if (id >= MN) return;");
  o.line(F("const int r = (int)(id / %d), c = (int)(id - (i64)r * %d);", g.N, g.N));
  o.line("real v = part[id];");
  o.line("for (int z = 1; z < nsplit; ++z) v += part[(i64)z * MN + id];");
  o.line(g.store);
  o.close();
}

void uvw_prelude_extra(Out& o, const Plan& p) {
  o.line("struct __attribute__((aligned(16))) Q4 { real a, b, c, d; };  // four consecutive elements");
  if (p.dtype == CGTP_F64) {
    o.line("typedef double acc4 __attribute__((ext_vector_type(4)));");
    o.line("#define MFMA(a, b, c) __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0)");
    o.line("#define ROWOF(lane, rr) (4 * (rr) + ((lane) >> 4))");
  } else {
    o.line("typedef float acc4 __attribute__((ext_vector_type(4)));");
    o.line("#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0)");
    o.line("#define ROWOF(lane, rr) (4 * ((lane) >> 4) + (rr))");
  }
}

const char* kStateArgs =
    "const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ G,"
    " const int* __restrict__ row_ptr, const int* __restrict__ col, real* __restrict__ S";

// Receiver state of task T for one receiver (Sobek Eq. 33): rows (il, m3), columns (pi, q, u).
void emit_state_task(Out& o, const Plan& p, const std::vector<Side>& sides, int ti, const StateTask& T,
                     const std::vector<size_t>& side_off, long long node_stride) {
  const Side& S = sides[T.side];
  const int K = p.K, d3 = S.d;
  std::vector<int> paths;
  for (int k : T.idx) paths.push_back(S.paths[k]);
  o.open(F("DEV void uvs_t%d(%s, int node, int il, int e_base, int w, int nst, real* sm)", ti, kStateArgs));
  o.line("const int lane = (int)threadIdx.x & 63;");
  o.line(F("const int u = %d + lane;", T.cb * 64));
  for (int b : in_blocks_of(p, paths)) o.line(F("const int uc%d = u < %d ? u : %d;", b, p.in[b].mul, p.in[b].mul - 1));
  std::vector<std::string> acc;
  for (int pi : paths)
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d3; ++m) {
        acc.push_back(F("s%d_%d_%d", pi, q, m));
        o.line("real " + acc.back() + " = R(0);");
      }
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  emit_recv_edge_loop(o, p, in_blocks_of(p, paths), "w", "nst", [&] {
    for (int pi : paths) {
      const Path& P = p.paths[pi];
      std::vector<bool> started(d3, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (!started[m3])
          o.line(F("real t%d_%d = g[%d] * x%d_%d;", pi, m3, P.g_off + int(t), P.i_in, m1));
        else
          o.line(F("t%d_%d = fma(g[%d], x%d_%d, t%d_%d);", pi, m3, P.g_off + int(t), P.i_in, m1, pi, m3));
        started[m3] = true;
      }
      for (int q = 0; q < K; ++q)
        for (int m = 0; m < d3; ++m)
          if (started[m]) o.line(F("s%d_%d_%d = fma(f%d, t%d_%d, s%d_%d_%d);", pi, q, m, q, pi, m, pi, q, m));
    }
  }, true);
  // The nst waves of the workgroup took every nst-th edge: partial states summed in LDS in a fixed
  // order (wave 0 first, then 1, ...).
  const int n = int(acc.size());
  o.open("if (nst > 1)");
  o.open("if (w != 0)");
  for (int m = 0; m < n; ++m) o.line(F("sm[((w - 1) * %d + %d) * 64 + lane] = %s;", n, m, acc[m].c_str()));
  o.close();
  o.line("__syncthreads();");
  o.open("if (w == 0)");
  o.open("for (int k = 1; k < nst; ++k)");
  for (int m = 0; m < n; ++m) o.line(F("%s += sm[((k - 1) * %d + %d) * 64 + lane];", acc[m].c_str(), n, m));
  o.close();
  o.close();
  o.close();
  o.line("if (w != 0) return;");
  for (size_t kk = 0; kk < T.idx.size(); ++kk) {
    const int k = T.idx[kk], pi = S.paths[k], mul = S.cmul[k];
    o.open(F("if (u < %d)", mul));
    o.line(F("real* __restrict__ dst = S + %zu + (i64)il * %lld + %d + u;", side_off[T.side], node_stride, S.col_off[k]));
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d3; ++m) o.line(F("dst[%d] = s%d_%d_%d;", m * S.ld + q * mul, pi, q, m));
    o.close();
  }
  o.close();
}

// One wave per (task, receiver); XCD-contiguous receiver ranges as in the channelwise forward.
// nst waves per workgroup split the receiver's edge list (nst = blockDim.x / 64, at most
// kMaxStripes); their partial states meet in dynamic LDS of (nst - 1) x state_acc x 64 values.
void emit_state_dispatch(Out& o, int ntask) {
  o.line(F("extern \"C\" __global__ void __launch_bounds__(%d)", 64 * kMaxStripes));
  o.open(std::string("cgtp_uvw_state(") + kStateArgs + ", int i0, int nrec, int per, int e_base)");
  o.line("extern __shared__ real sm[];");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, il = xcd * per + (s - t * per);");
  o.line("if (il >= nrec) return;");
  o.line("const int nst = (int)blockDim.x >> 6, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);");
  o.open("switch (t)");
  for (int k = 0; k < ntask; ++k)
    o.line(F("case %d: uvs_t%d(x, phi, G, row_ptr, col, S, i0 + il, il, e_base, w, nst, sm); break;", k, k));
  o.line("default: break;");
  o.close();
  o.close();
}

const char* kEdgeArgs =
    "const real* __restrict__ x, const real* __restrict__ phi, const real* __restrict__ G,"
    " const int* __restrict__ row_ptr, const int* __restrict__ col, const real* __restrict__ Sb,"
    " real* __restrict__ ep";

// Per-edge backward of task T (receiver side): phi-bar_q = sum_{pi,m3} Sbar[pi][q][m3] C_pi[m3] and
// Y-bar from Cbar[pi][m3] = sum_q phi_q Sbar[pi][q][m3], both reduced over the channels of the wave
// into the edge's partial columns of task ti.
void emit_edge_task(Out& o, const Plan& p, const std::vector<Side>& sides, int ti, const StateTask& T,
                    const std::vector<size_t>& side_off, long long node_stride, int V) {
  const Side& S = sides[T.side];
  const int K = p.K, d3 = S.d;
  std::vector<int> paths;
  for (int k : T.idx) paths.push_back(S.paths[k]);
  // NST = 1: one wave per receiver (constant stride, the common case); NST = 0: stride nst.
  o.line("template <int NST>");
  o.open(F("DEV void uve_t%d(%s, int node, int il, int e_base, int eps, int stripe, int nst)", ti, kEdgeArgs));
  o.line("const int st_ = NST == 1 ? 0 : stripe, ns_ = NST == 1 ? 1 : nst;");
  o.line("const int lane = (int)threadIdx.x & 63;");
  o.line(F("const int u = %d + lane;", T.cb * 64));
  for (int b : in_blocks_of(p, paths)) o.line(F("const int uc%d = u < %d ? u : %d;", b, p.in[b].mul, p.in[b].mul - 1));
  for (size_t kk = 0; kk < T.idx.size(); ++kk) {
    const int k = T.idx[kk], pi = S.paths[k], mul = S.cmul[k];
    o.line(F("const real* __restrict__ sr%d = Sb + %zu + (i64)il * %lld + %d + (u < %d ? u : 0);", pi,
             side_off[T.side], node_stride, S.col_off[k], mul));
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d3; ++m)
        o.line(F("const real sb%d_%d_%d = u < %d ? sr%d[%d] : R(0);", pi, q, m, mul, pi, m * S.ld + q * mul));
  }
  o.line("const int e0 = row_ptr[node], e1 = row_ptr[node + 1];");
  emit_recv_edge_loop(o, p, in_blocks_of(p, paths), "st_", "ns_", [&] {
    for (int v = 0; v < V; ++v) o.line(F("real v%d = R(0);", v));
    for (int pi : paths) {
      const Path& P = p.paths[pi];
      const int s = K + P.l2 * P.l2;
      std::vector<bool> started(d3, false);
      for (size_t t = 0; t < P.gpairs.size(); ++t) {
        int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
        if (!started[m3])
          o.line(F("real t%d_%d = g[%d] * x%d_%d;", pi, m3, P.g_off + int(t), P.i_in, m1));
        else
          o.line(F("t%d_%d = fma(g[%d], x%d_%d, t%d_%d);", pi, m3, P.g_off + int(t), P.i_in, m1, pi, m3));
        started[m3] = true;
      }
      for (int q = 0; q < K; ++q)
        for (int m = 0; m < d3; ++m)
          if (started[m]) o.line(F("v%d = fma(sb%d_%d_%d, t%d_%d, v%d);", q, pi, q, m, pi, m, q));
      std::set<int> m3used;
      for (auto& gp : P.gpairs) m3used.insert(gp.m3);
      for (int m : m3used) {
        o.line(F("real cb%d_%d = f0 * sb%d_0_%d;", pi, m, pi, m));
        for (int q = 1; q < K; ++q) o.line(F("cb%d_%d = fma(f%d, sb%d_%d_%d, cb%d_%d);", pi, m, q, pi, q, m, pi, m));
      }
      for (auto& gp : P.gpairs) {
        o.line(F("{ const real z = x%d_%d * cb%d_%d;", P.i_in, gp.m1, pi, gp.m3));
        for (auto& t : gp.terms)
          o.line(F("  v%d = fma(%s, z, v%d);", s + t.first, lit(t.second).c_str(), s + t.first));
        o.line("}");
      }
    }
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
        return F("ep[(i64)(%d + r_ * %d + ", ti * V, Q) + kk + ") * eps + (e - e_base)] = " + val + ";";
      });
      return;
    }
    for (int k = 0; k < Q; ++k) o.line(F("v%d = rowsum(v%d);", k, k));
    o.open("if ((lane & 15) == 0)");
    o.line(F("real* __restrict__ dst = ep + (i64)(%d + (lane >> 4) * %d) * eps + (e - e_base);", ti * V, Q));
    for (int k = 0; k < Q; ++k) o.line(F("dst[(i64)%d * eps] = v%d;", k, k));
    o.close();
  }, true);
  o.close();
}

// One wave per (task, receiver, stripe): the nst stripes of a receiver take every nst-th edge
// (per-edge outputs, nothing to combine).
void emit_edge_dispatch(Out& o, int ntask) {
  // cgtp_uvw_edge: one wave per (task, receiver); cgtp_uvw_edge_striped: nst waves per receiver
  // (separate kernels so that each gets its own register allocation).
  for (int striped = 0; striped < 2; ++striped) {
    o.line("extern \"C\" __global__ void __launch_bounds__(64)");
    o.open(std::string(striped ? "cgtp_uvw_edge_striped(" : "cgtp_uvw_edge(") + kEdgeArgs +
           ", int i0, int nrec, int per, int e_base, int eps, int nst)");
    o.line("const int b = (int)blockIdx.x;");
    o.line("const int xcd = b & 7, s = b >> 3;");
    o.line("const int t = s / (per * nst), r = s - t * per * nst;");
    o.line("const int il = xcd * per + r / nst, stripe = r - (r / nst) * nst;");
    o.line("if (il >= nrec) return;");
    o.open("switch (t)");
    for (int k = 0; k < ntask; ++k)
      o.line(F("case %d: uve_t%d<%d>(x, phi, G, row_ptr, col, Sb, ep, i0 + il, il, e_base, eps, stripe, nst); break;",
               k, k, striped ? 0 : 1));
    o.line("default: break;");
    o.close();
    o.close();
  }
}

const char* kZArgs =
    "const real* __restrict__ phi, const real* __restrict__ G, const real* __restrict__ gout,"
    " const int* __restrict__ recv, const int* __restrict__ src_ptr, const int* __restrict__ src_edge,"
    " real* __restrict__ Z";

// Source-side state of task T for one sender j: rows (jl, m1), columns (pi, q, w), with G rows
// stored in source-CSR order (row k - k_base for out-edge position k).
void emit_zstate_task(Out& o, const Plan& p, const std::vector<Side>& sides, int ti, const StateTask& T,
                      const std::vector<size_t>& side_off, long long node_stride) {
  const Side& S = sides[T.side];
  const int K = p.K, d1 = S.d;
  std::vector<int> paths;
  for (int k : T.idx) paths.push_back(S.paths[k]);
  const auto obs = out_blocks_of(p, paths);
  o.open(F("DEV void uvz_t%d(%s, int node, int jl, int k_base)", ti, kZArgs));
  o.line("const int lane = (int)threadIdx.x & 63;");
  o.line(F("const int w = %d + lane;", T.cb * 64));
  for (int ob : obs) o.line(F("const int wc%d = w < %d ? w : %d;", ob, p.out[ob].mul, p.out[ob].mul - 1));
  for (int pi : paths)
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d1; ++m) o.line(F("real z%d_%d_%d = R(0);", pi, q, m));
  o.line("const int s0 = src_ptr[node], s1 = src_ptr[node + 1];");
  // Edge ids and receivers of up to 64 out-edges, one per lane, taken one by one with readlane.
  o.open("for (int kb_ = s0; kb_ < s1; kb_ += 64)");
  o.line("const int kl_ = kb_ + lane;");
  o.line("const int el_ = src_edge[kl_ < s1 ? kl_ : kb_];");
  o.line("const int il_ = recv[el_];");
  o.line("const int ne_ = min(64, s1 - kb_);");
  o.open("for (int k_ = 0; k_ < ne_; ++k_)");
  o.line("const int k = kb_ + k_;");
  o.line("const int e = __builtin_amdgcn_readlane(el_, k_);");
  o.line("const int i_ = __builtin_amdgcn_readlane(il_, k_);");
  for (int ob : obs) {
    const Block& B = p.out[ob];
    for (int m = 0; m < B.dim(); ++m)
      o.line(F("const real mb%d_%d = gout[(i64)i_ * %d + %d + wc%d];", ob, m, p.c_out, B.offset + m * B.mul, ob));
  }
  o.line(F("const real* __restrict__ g = G + (i64)(k - k_base) * %d;", p.g_stride));
  o.line("const real* __restrict__ ph = " + phi_ptr(p, "e", "g") + ";");
  for (int q = 0; q < K; ++q) o.line(F("const real f%d = ph[%d];", q, q));
  for (int pi : paths) {
    const Path& P = p.paths[pi];
    std::vector<bool> started(d1, false);
    for (size_t t = 0; t < P.gpairs.size(); ++t) {
      int m1 = P.gpairs[t].m1, m3 = P.gpairs[t].m3;
      if (!started[m1])
        o.line(F("real b%d_%d = g[%d] * mb%d_%d;", pi, m1, P.g_off + int(t), P.i_out, m3));
      else
        o.line(F("b%d_%d = fma(g[%d], mb%d_%d, b%d_%d);", pi, m1, P.g_off + int(t), P.i_out, m3, pi, m1));
      started[m1] = true;
    }
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d1; ++m)
        if (started[m]) o.line(F("z%d_%d_%d = fma(f%d, b%d_%d, z%d_%d_%d);", pi, q, m, q, pi, m, pi, q, m));
  }
  o.close();
  o.close();
  for (size_t kk = 0; kk < T.idx.size(); ++kk) {
    const int k = T.idx[kk], pi = S.paths[k], mul = S.cmul[k];
    o.open(F("if (w < %d)", mul));
    o.line(F("real* __restrict__ dst = Z + %zu + (i64)jl * %lld + %d + w;", side_off[T.side], node_stride, S.col_off[k]));
    for (int q = 0; q < K; ++q)
      for (int m = 0; m < d1; ++m) o.line(F("dst[%d] = z%d_%d_%d;", m * S.ld + q * mul, pi, q, m));
    o.close();
  }
  o.close();
}

void emit_zstate_dispatch(Out& o, int ntask) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open(std::string("cgtp_uvw_zstate(") + kZArgs + ", int j0, int njs, int per, int k_base)");
  o.line("const int b = (int)blockIdx.x;");
  o.line("const int xcd = b & 7, s = b >> 3;");
  o.line("const int t = s / per, jl = xcd * per + (s - t * per);");
  o.line("if (jl >= njs) return;");
  o.open("switch (t)");
  for (int k = 0; k < ntask; ++k)
    o.line(F("case %d: uvz_t%d(phi, G, gout, recv, src_ptr, src_edge, Z, j0 + jl, jl, k_base); break;", k, k));
  o.line("default: break;");
  o.close();
  o.close();
}

// G rows of the out-edges at source-CSR positions [k0, k1) (row k - k0 for edge src_edge[k]).
void emit_prep_src(Out& o, const Plan& p) {
  o.line("extern \"C\" __global__ void __launch_bounds__(64)");
  o.open("cgtp_prep_src(const real* __restrict__ pos, const real* __restrict__ shift, const int* __restrict__ recv,"
         " const int* __restrict__ send, const int* __restrict__ src_edge, int k0, int k1, real* __restrict__ G)");
  o.line("const int k = k0 + (int)(blockIdx.x * 64 + threadIdx.x);");
  o.line("if (k >= k1) return;");
  o.line("const int e = src_edge[k];");
  emit_edge_vector(o);
  o.line("const real rr = sqrt(rx * rx + ry * ry + rz * rz), inv = R(1) / rr;");
  o.line(F("real Y[%d];", p.sh_dim));
  o.line("sh_eval<real>(rx * inv, ry * inv, rz * inv, Y);");
  o.line(F("real* __restrict__ dst = G + (i64)(k - k0) * %d;", p.g_stride));
  if (p.radial) {
    o.line(F("real fr[%d];", p.K));
    o.line("radial_eval(rr, fr, nullptr, nullptr);");
    for (int q = 0; q < p.K; ++q) o.line(F("dst[%d] = fr[%d];", p.phi_off + q, q));
  }
  for (const Path& P : p.paths) {
    int s = P.l2 * P.l2;
    int n = P.g_off;
    for (const GPair& gp : P.gpairs) {
      std::string ex;
      for (auto& t : gp.terms) {
        if (!ex.empty()) ex += " + ";
        ex += lit(t.second) + " * Y[" + std::to_string(s + t.first) + "]";
      }
      o.line(F("dst[%d] = ", n++) + ex + ";");
    }
  }
  o.close();
}

// Per-node layout of a state: sides back to back, side g holding d_g rows of ld_g values.
std::vector<size_t> side_offsets(const std::vector<Side>& sides, long long* stride) {
  std::vector<size_t> off;
  size_t acc = 0;
  for (auto& s : sides) {
    off.push_back(acc);
    acc += size_t(s.d) * size_t(s.ld);
  }
  *stride = (long long)acc;
  return off;
}

// Address of row r (node r / d, component r % d), column `col` of side s of a per-node state.
std::string state_at(const std::string& base, const Side& s, size_t off, long long stride, const std::string& r,
                     const std::string& col) {
  return F("%s[(i64)(%s / %d) * %lld + %zu + (%s %% %d) * %d + %s]", base.c_str(), r.c_str(), s.d, stride, off,
           r.c_str(), s.d, s.ld, col.c_str());
}

}  // namespace

// Layout facts the launcher needs (columns, strides, task counts).
UvwLayout uvw_layout(const Plan& p) {
  UvwLayout L;
  auto rs = recv_sides(p), ss = send_sides(p);
  for (auto& s : rs) L.recv.push_back({s.blk, s.d, s.mul, s.D, s.ld});
  for (auto& s : ss) L.send.push_back({s.blk, s.d, s.mul, s.D, s.ld});
  side_offsets(rs, &L.recv_stride);
  side_offsets(ss, &L.send_stride);
  const auto st = state_tasks(p, rs, recv_state_cost);
  L.n_state_tasks = int(st.size());
  for (const StateTask& t : st) L.state_acc = std::max(L.state_acc, int(t.idx.size()) * p.K * rs[t.side].d);
  L.n_z_tasks = int(state_tasks(p, ss, send_state_cost).size());
  return L;
}

std::string generate_uvw_source(const Plan& p, const std::string& family, std::string* err) {
  if (family != "uvw_fwd" && family != "uvw_bwd" && family != "uvw_dbl") {
    *err = "the fully connected mode supports the streamed schedule only (family " + family + ")";
    return "";
  }
  // uvw_dbl: the backward's kernels, the forward GEMMs and the double backward's own kernels.
  const bool dbl = family == "uvw_dbl";
  const bool bwd = family != "uvw_fwd";
  Out o;
  prelude(o, p, bwd, bwd);
  uvw_prelude_extra(o, p);
  emit_sh(o, p.lmax);
  emit_prep(o, p);
  if (!bwd) emit_check_edges(o);
  auto rs = recv_sides(p);
  long long RS = 0;
  const std::vector<size_t> roff = side_offsets(rs, &RS);
  auto st = state_tasks(p, rs, recv_state_cost);
  for (int k = 0; k < int(st.size()); ++k) emit_state_task(o, p, rs, k, st[k], roff, RS);
  emit_state_dispatch(o, int(st.size()));
  for (auto& s : rs) {
    emit_brow(o, p, s, F("brow%d", s.blk));
  }
  if (!bwd || dbl) {
    for (size_t gi = 0; gi < rs.size(); ++gi) {
      const Side& s = rs[gi];
      const Block& OB = p.out[s.blk];
      GemmSpec g;
      g.name = F("cgtp_gemm_fwd%d", s.blk);
      g.args = "const real* __restrict__ S, const real* __restrict__ A, real* __restrict__ part, int i0";
      g.a_at = state_at("S", s, roff[gi], RS, "r", "k");
      g.b_at = F("A[brow%d(k) + c]", s.blk);
      g.store = F("part[(i64)blockIdx.z * M * %d + (i64)r * %d + c] = v;", OB.mul, OB.mul);
      g.N = OB.mul;
      g.a_kfast = true;
      g.b_kfast = false;
      g.split = true;
      g.vec = gemm_vec_ok(p);
      g.a_ptr = "S";
      g.b_ptr = "A";
      emit_gemm(o, g);
      g.store = F("out[(i64)(i0 + r / %d) * %d + %d + (r %% %d) * %d + c] = v;", s.d, p.c_out, OB.offset, s.d, OB.mul);
      emit_gemm_reduce(o, g, "real* __restrict__ out, int i0");
    }
    if (!bwd) return o.s.str();
  }
  // ---- backward
  for (size_t gi = 0; gi < rs.size(); ++gi) {
    const Side& s = rs[gi];
    const Block& OB = p.out[s.blk];
    GemmSpec g;  // Sbar = mbar A^T
    g.name = F("cgtp_gemm_sbar%d", s.blk);
    g.args = "const real* __restrict__ gout, const real* __restrict__ A, real* __restrict__ Sb, int i0";
    g.a_at = F("gout[(i64)(i0 + r / %d) * %d + %d + (r %% %d) * %d + k]", s.d, p.c_out, OB.offset, s.d, OB.mul);
    g.b_at = F("A[brow%d(c) + k]", s.blk);
    g.store = state_at("Sb", s, roff[gi], RS, "r", "c") + " = v;";
    g.N = s.D;
    g.a_kfast = true;
    g.b_kfast = true;
    g.split = false;
    g.vec = gemm_vec_ok(p);
    g.a_ptr = "gout";
    g.b_ptr = "A";
    if (sbar_panel(OB.mul))
      emit_gemm_panel(o, g);
    else
      emit_gemm(o, g);
    GemmSpec h;  // A-bar partials = S^T mbar over a slice of rows
    h.name = F("cgtp_gemm_abar%d", s.blk);
    h.args = "const real* __restrict__ S, const real* __restrict__ gout, real* __restrict__ part, int i0";
    h.a_at = state_at("S", s, roff[gi], RS, "k", "r");
    h.b_at = F("gout[(i64)(i0 + k / %d) * %d + %d + (k %% %d) * %d + c]", s.d, p.c_out, OB.offset, s.d, OB.mul);
    h.store = F("part[(i64)blockIdx.z * %lld + (i64)r * %d + c] = v;", (long long)s.D * OB.mul, OB.mul);
    h.N = OB.mul;
    h.a_kfast = false;
    h.b_kfast = false;
    h.split = true;
    h.vec = gemm_vec_ok(p);
    h.a_ptr = "S";
    h.b_ptr = "gout";
    emit_gemm(o, h);
    // A-bar += sum over row slices (fixed order), scattered into the layout of A.
    o.line("extern \"C\" __global__ void __launch_bounds__(256)");
    o.open(F("cgtp_abar_accum%d(const real* __restrict__ part, int nsplit, real* __restrict__ gA)", s.blk));
    o.line(F("const int id = (int)(blockIdx.x * 256 + threadIdx.x);"));
    o.line(F("if (id >= %d) return;", s.D * OB.mul));
    o.line(F("const int r = id / %d, c = id - r * %d;", OB.mul, OB.mul));
    o.line("real acc = R(0);");
    o.line(F("for (int k = 0; k < nsplit; ++k) acc += part[(i64)k * %d + id];", s.D * OB.mul));
    o.line(F("gA[brow%d(r) + c] += acc;", s.blk));
    o.close();
  }
  const int V = edge_partial_width(p);
  for (int k = 0; k < int(st.size()); ++k) emit_edge_task(o, p, rs, k, st[k], roff, RS, V);
  emit_edge_dispatch(o, int(st.size()));
  emit_edge_final(o, p, int(st.size()), V);
  emit_small_kernels(o);
  // source side
  emit_prep_src(o, p);
  auto ss = send_sides(p);
  auto zt = state_tasks(p, ss, send_state_cost);
  long long ZS = 0;
  const std::vector<size_t> zoff = side_offsets(ss, &ZS);
  for (int k = 0; k < int(zt.size()); ++k) emit_zstate_task(o, p, ss, k, zt[k], zoff, ZS);
  emit_zstate_dispatch(o, int(zt.size()));
  for (size_t bi = 0; bi < ss.size(); ++bi) {
    const Side& s = ss[bi];
    const Block& IB = p.in[s.blk];
    emit_bz(o, p, s, F("bz%d", s.blk));
    GemmSpec g;  // x-bar = Z A (contracting (pi, q, w))
    g.name = F("cgtp_gemm_xbar%d", s.blk);
    g.args = "const real* __restrict__ Z, const real* __restrict__ A, real* __restrict__ part, int j0";
    g.a_at = state_at("Z", s, zoff[bi], ZS, "r", "k");
    g.b_at = F("A[bxi%d(k, c)]", s.blk);
    g.store = F("part[(i64)blockIdx.z * M * %d + (i64)r * %d + c] = v;", IB.mul, IB.mul);
    g.N = IB.mul;
    g.a_kfast = true;
    g.b_kfast = true;
    g.split = true;
    g.vec = gemm_vec_ok(p);
    g.a_ptr = "Z";
    g.b_ptr = "A";
    o.line(F("DEV i64 bxi%d(int k, int c) { int st; const i64 b = bz%d(k, st); return b + (i64)c * st; }", s.blk,
             s.blk));
    emit_gemm(o, g);
    g.store = F("gx[(i64)(j0 + r / %d) * %d + %d + (r %% %d) * %d + c] = v;", s.d, p.c_in, IB.offset, s.d, IB.mul);
    emit_gemm_reduce(o, g, "real* __restrict__ gx, int j0");
  }
  if (dbl) emit_uvw_dbl_kernels(o, p, int(st.size()), V);
  return o.s.str();
}

}  // namespace cgtp
