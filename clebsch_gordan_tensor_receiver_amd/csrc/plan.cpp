// Plan construction: irreps parsing, path enumeration and the real Clebsch-Gordan tables.
//
// Path rule (Sobek, section 2.2, Eq. 5): |l1 - l2| <= l3 <= l1 + l2 and
// parity_out = parity_in * parity_sh; channelwise paths also tie mul_in = mul_out
// (section 2.3, Eq. 6).  Weight counts n_pi = C (channelwise) or C_in C_out (fully
// connected) and N_w = sum n_pi (section 2.4, Eqs. 8-9).
//
// Coupling coefficients (LunaTP, section 2.1, Eq. 1): complex CG from the Racah closed-form
// sum, moved to the basis of the real spherical harmonics and made sign-definite (first
// non-zero entry of each tensor positive).
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <complex>
#include <sstream>

#include "kernels.hpp"

namespace cgtp {

Plan::~Plan() = default;

bool parse_irreps(const std::string& s, std::vector<Block>* out, std::string* err) {
  out->clear();
  int off = 0;
  size_t i = 0;
  std::string t;
  for (char ch : s)
    if (ch != ' ') t.push_back(ch);
  if (t.empty()) {
    *err = "empty irreps string";
    return false;
  }
  while (i <= t.size()) {
    size_t j = t.find('+', i);
    if (j == std::string::npos) j = t.size();
    std::string tok = t.substr(i, j - i);
    size_t x = tok.find('x');
    if (x == std::string::npos || x == 0 || x + 2 > tok.size()) {
      *err = "bad irreps token '" + tok + "'";
      return false;
    }
    char p = tok.back();
    std::string mul_s = tok.substr(0, x), l_s = tok.substr(x + 1, tok.size() - x - 2);
    if ((p != 'e' && p != 'o') || l_s.empty() ||
        mul_s.find_first_not_of("0123456789") != std::string::npos ||
        l_s.find_first_not_of("0123456789") != std::string::npos || mul_s.size() > 6 || l_s.size() > 3) {
      *err = "bad irreps token '" + tok + "'";
      return false;
    }
    Block b;
    b.mul = std::stoi(mul_s);
    b.l = std::stoi(l_s);
    b.parity = p == 'e' ? 1 : -1;
    b.offset = off;
    if (b.mul < 1) {
      *err = "multiplicity must be positive in '" + tok + "'";
      return false;
    }
    off += b.size();
    out->push_back(b);
    i = j + 1;
  }
  return true;
}

static long double fact(int n) {
  long double r = 1;
  for (int k = 2; k <= n; ++k) r *= k;
  return r;
}

long double complex_cg(int l1, int m1, int l2, int m2, int l3, int m3) {
  if (m3 != m1 + m2) return 0;
  if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return 0;
  if (std::abs(m1) > l1 || std::abs(m2) > l2 || std::abs(m3) > l3) return 0;
  long double pre = (2 * l3 + 1) * fact(l3 + l1 - l2) * fact(l3 - l1 + l2) * fact(l1 + l2 - l3) /
                    fact(l1 + l2 + l3 + 1);
  pre *= fact(l3 + m3) * fact(l3 - m3) * fact(l1 - m1) * fact(l1 + m1) * fact(l2 - m2) * fact(l2 + m2);
  long double s = 0, smax = 0;
  for (int k = 0; k <= l1 + l2 + l3; ++k) {
    int d[6] = {k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k};
    bool ok = true;
    long double den = 1;
    for (int v : d) {
      if (v < 0) ok = false;
      else den *= fact(v);
    }
    if (!ok) continue;
    long double term = ((k & 1) ? -1.0L : 1.0L) / den;
    s += term;
    smax = std::max(smax, std::fabs(term));
  }
  if (std::fabs(s) <= 1e-15L * smax) return 0;  // exact cancellation (an accidental zero)
  return s * std::sqrt(pre);
}

// Complex-to-real change of basis: Y_real[mu] = sum_m U(mu, m) Y_complex[m].
//   mu > 0: ((-1)^mu Y^mu + Y^-mu) / sqrt2,  mu = 0: Y^0,  mu < 0: i (Y^mu - (-1)^|mu| Y^|mu|) / sqrt2.
// Returns the (at most two) non-zero entries of row mu as (m, value).
static int basis_row(int mu, std::pair<int, std::complex<long double>> ent[2]) {
  const long double r = 1.0L / std::sqrt(2.0L);
  if (mu == 0) {
    ent[0] = {0, {1.0L, 0.0L}};
    return 1;
  }
  if (mu > 0) {
    ent[0] = {mu, {(mu & 1) ? -r : r, 0.0L}};
    ent[1] = {-mu, {r, 0.0L}};
    return 2;
  }
  int a = -mu;
  ent[0] = {mu, {0.0L, r}};
  ent[1] = {a, {0.0L, (a & 1) ? r : -r}};
  return 2;
}

std::vector<double> real_cg(int l1, int l2, int l3) {
  int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
  std::vector<std::complex<long double>> c(size_t(d1) * d2 * d3);
  std::pair<int, std::complex<long double>> e1[2], e2[2], e3[2];
  for (int a = 0; a < d1; ++a) {
    int n1 = basis_row(a - l1, e1);
    for (int b = 0; b < d2; ++b) {
      int n2 = basis_row(b - l2, e2);
      for (int k = 0; k < d3; ++k) {
        int n3 = basis_row(k - l3, e3);
        std::complex<long double> acc = 0;
        for (int i = 0; i < n1; ++i)
          for (int j = 0; j < n2; ++j)
            for (int q = 0; q < n3; ++q) {
              long double v = complex_cg(l1, e1[i].first, l2, e2[j].first, l3, e3[q].first);
              if (v == 0) continue;
              acc += e3[q].second * std::conj(e1[i].second) * std::conj(e2[j].second) * v;
            }
        c[(size_t(a) * d2 + b) * d3 + k] = acc;
      }
    }
  }
  long double re = 0, im = 0;
  for (auto& v : c) {
    re = std::max(re, std::fabs(v.real()));
    im = std::max(im, std::fabs(v.imag()));
  }
  bool use_re = re >= im;
  std::vector<double> out(c.size());
  for (size_t i = 0; i < c.size(); ++i) {
    long double v = use_re ? c[i].real() : c[i].imag();
    out[i] = std::fabs(v) < 1e-13L ? 0.0 : double(v);
  }
  for (double v : out)
    if (v != 0.0) {
      if (v < 0)
        for (double& w : out) w = -w;
      break;
    }
  for (double& w : out)
    if (w == 0.0) w = 0.0;  // no negative zeros
  return out;
}

cgtp_status_t build_plan(const char* irreps_in, const char* irreps_sh, const char* irreps_out,
                         cgtp_mode_t mode, cgtp_dtype_t dtype, int K, Plan* p, std::string* err) {
  if (!irreps_in || !irreps_sh || !irreps_out) {
    *err = "null irreps string";
    return CGTP_ERR_INVALID_ARG;
  }
  if (mode != CGTP_CHANNELWISE && mode != CGTP_FULLY_CONNECTED) {
    *err = "unknown mode";
    return CGTP_ERR_INVALID_ARG;
  }
  if (dtype != CGTP_F32 && dtype != CGTP_F64) {
    *err = "unknown dtype";
    return CGTP_ERR_INVALID_ARG;
  }
  if (K < 1 || K > 64) {
    *err = "num_radial must be in [1, 64]";
    return CGTP_ERR_INVALID_ARG;
  }
  if (!parse_irreps(irreps_in, &p->in, err) || !parse_irreps(irreps_sh, &p->sh, err) ||
      !parse_irreps(irreps_out, &p->out, err))
    return CGTP_ERR_INVALID_ARG;
  for (size_t k = 0; k < p->sh.size(); ++k) {
    const Block& b = p->sh[k];
    // The parity label of an edge block (normally (-1)^l) only enters path selection: the values
    // are always the real spherical harmonics (LunaTP's C1 profile labels degree 1 "1e").
    if (b.mul != 1 || b.l != int(k)) {
      *err = "spherical-harmonic irreps must be 1x0e+1x1?+...+1xL? (one block per degree, in order)";
      return CGTP_ERR_INVALID_ARG;
    }
  }
  for (const auto* v : {&p->in, &p->sh, &p->out})
    for (const Block& b : *v)
      if (b.l > kMaxL) {
        *err = "degrees above 6 are not supported";
        return CGTP_ERR_UNSUPPORTED;
      }
  p->mode = mode;
  p->dtype = dtype;
  p->K = K;
  p->lmax = int(p->sh.size()) - 1;
  p->sh_dim = (p->lmax + 1) * (p->lmax + 1);
  p->c_in = p->c_out = 0;
  for (auto& b : p->in) p->c_in += b.size();
  for (auto& b : p->out) p->c_out += b.size();
  int w_off = 0, g_off = 0, nnz = 0;
  for (int i = 0; i < int(p->in.size()); ++i)
    for (int j = 0; j < int(p->sh.size()); ++j)
      for (int k = 0; k < int(p->out.size()); ++k) {
        const Block &a = p->in[i], &s = p->sh[j], &o = p->out[k];
        if (o.l < std::abs(a.l - s.l) || o.l > a.l + s.l) continue;
        if (a.parity * s.parity != o.parity) continue;
        if (mode == CGTP_CHANNELWISE && a.mul != o.mul) continue;
        Path P;
        P.i_in = i;
        P.i_sh = j;
        P.i_out = k;
        P.l1 = a.l;
        P.l2 = s.l;
        P.l3 = o.l;
        P.w_off = w_off;
        P.n_w = mode == CGTP_CHANNELWISE ? a.mul : a.mul * o.mul;
        w_off += P.n_w;
        std::vector<double> c = real_cg(a.l, s.l, o.l);
        int d1 = a.dim(), d2 = s.dim(), d3 = o.dim();
        for (int m1 = 0; m1 < d1; ++m1)
          for (int m2 = 0; m2 < d2; ++m2)
            for (int m3 = 0; m3 < d3; ++m3) {
              double v = c[(size_t(m1) * d2 + m2) * d3 + m3];
              if (v != 0.0) P.terms.push_back({m1, m2, m3, v});
            }
        for (int m3 = 0; m3 < d3; ++m3)
          for (int m1 = 0; m1 < d1; ++m1) {
            GPair gp{m1, m3, {}};
            for (int m2 = 0; m2 < d2; ++m2) {
              double v = c[(size_t(m1) * d2 + m2) * d3 + m3];
              if (v != 0.0) gp.terms.push_back({m2, v});
            }
            if (!gp.terms.empty()) P.gpairs.push_back(gp);
          }
        nnz += int(P.terms.size());
        p->paths.push_back(std::move(P));
      }
  if (p->paths.empty()) {
    *err = "no admissible path between these irreps";
    return CGTP_ERR_UNSUPPORTED;
  }
  // G layout: the paths' (m1, m3) pairs back to back.  Plans with large paths read those through
  // 16-byte vector loads, so their path blocks start on multiples of 4 values.
  p->vec_g = false;
  for (const Path& P : p->paths) p->vec_g = p->vec_g || int(P.gpairs.size()) > kVecGPairs;
  for (Path& P : p->paths) {
    if (p->vec_g) g_off = (g_off + 3) / 4 * 4;
    P.g_off = g_off;
    g_off += int(P.gpairs.size());
  }
  p->n_w = w_off;
  p->g_width = g_off;
  p->g_stride = (g_off + 3) / 4 * 4;
  p->cg_nnz = nnz;
  p->by_out.assign(p->out.size(), {});
  p->by_in.assign(p->in.size(), {});
  for (int k = 0; k < int(p->paths.size()); ++k) {
    p->by_out[p->paths[k].i_out].push_back(k);
    p->by_in[p->paths[k].i_in].push_back(k);
  }
  std::ostringstream key;
  key << "v1|" << irreps_in << "|" << irreps_sh << "|" << irreps_out << "|" << int(mode) << "|"
      << int(dtype) << "|" << K;
  p->key = key.str();
  p->irreps_in_s = irreps_in;
  p->irreps_sh_s = irreps_sh;
  p->irreps_out_s = irreps_out;
  p->kernels = make_kernel_set();
  return CGTP_OK;
}

}  // namespace cgtp
