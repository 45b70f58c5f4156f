// Host-side derivation of the 3-bit magnitude codebook of ParisKV's 4-bit
// direction codes (ParisKV close-reading, section 2.4, paper Prop. 4.1 and
// App. B.1): with a Haar-random rotation, a coordinate u_j of a unit
// m-dimensional subspace direction has (u_j)^2 ~ Beta(1/2, (m-1)/2), so
// y = |u_j| has density proportional to (1 - y^2)^((m-3)/2) on [0, 1].  The
// eight reconstruction levels are the Lloyd-Max (minimum squared error)
// quantiser of that density: thresholds are midpoints of neighbouring levels,
// each level is the conditional mean of its cell, iterated to a fixed point in
// float64 and rounded once to fp32.
//
// Cell masses use the substitution y = sin(theta), which turns the integrand
// into cos(theta)^(m-2) (smooth, so composite Gauss-Legendre converges
// geometrically); first moments use the closed form
// integral y (1-y^2)^a dy = -(1-y^2)^(a+1) / (2(a+1)).
#include <math.h>

#include "../../include/sparsekv.h"

namespace {

// 10-point Gauss-Legendre nodes / weights on [-1, 1].
const double kGLx[5] = {0.1488743389816312108848260, 0.4333953941292471907992659,
                        0.6794095682990244062343274, 0.8650633666889845107320967,
                        0.9739065285171717200779640};
const double kGLw[5] = {0.2955242247147528701738930, 0.2692667193099963550912269,
                        0.2190863625159820439955349, 0.1494513491505805931457763,
                        0.0666713443086881375935688};

double mass(double t1, double t2, double a) {
  // integral_{t1}^{t2} (1 - y^2)^a dy = integral cos(th)^(2a+1) dth over [asin t1, asin t2]
  const double th1 = asin(t1), th2 = asin(t2);
  const int panels = 64;
  const double h = (th2 - th1) / panels;
  double sum = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double c = th1 + (p + 0.5) * h, r = 0.5 * h;
    for (int i = 0; i < 5; ++i) {
      sum += kGLw[i] * r * pow(cos(c - r * kGLx[i]), 2.0 * a + 1.0);
      sum += kGLw[i] * r * pow(cos(c + r * kGLx[i]), 2.0 * a + 1.0);
    }
  }
  return sum;
}

double moment(double t1, double t2, double a) {
  return (pow(1.0 - t1 * t1, a + 1.0) - pow(1.0 - t2 * t2, a + 1.0)) / (2.0 * (a + 1.0));
}

}  // namespace

extern "C" skv_status sparsekv_codebook_init(int32_t m, float levels[8], float thresh[7]) {
  if (!levels || !thresh || m < 3 || m > 16) return SKV_EINVAL;
  const double a = (m - 3) / 2.0;
  double lv[8], th[7], edges[9];
  for (int i = 0; i < 8; ++i) lv[i] = (i + 0.5) / 8.0;
  for (int it = 0; it < 20000; ++it) {
    edges[0] = 0.0;
    edges[8] = 1.0;
    for (int i = 0; i < 7; ++i) edges[i + 1] = 0.5 * (lv[i] + lv[i + 1]);
    double delta = 0.0;
    for (int i = 0; i < 8; ++i) {
      const double nl = moment(edges[i], edges[i + 1], a) / mass(edges[i], edges[i + 1], a);
      delta = fmax(delta, fabs(nl - lv[i]));
      lv[i] = nl;
    }
    if (delta <= 1e-15) break;
  }
  for (int i = 0; i < 7; ++i) th[i] = 0.5 * (lv[i] + lv[i + 1]);
  for (int i = 0; i < 8; ++i) levels[i] = (float)lv[i];
  for (int i = 0; i < 7; ++i) thresh[i] = (float)th[i];
  return SKV_OK;
}
