/* NVFP4 block-scale search of oracle/nvfp4.py written as plain C loops, for
 * tensors too large for the numpy version to finish in seconds.
 *
 * TEST INFRASTRUCTURE ONLY (see the oracle package header). Same definition
 * as oracle/nvfp4.py (reading R20 there): for each block of 16 magnitudes a
 * and each E4M3 code c = 1..126 with S = e4m3(c) * g, every element rounds to
 * the nearest E2M1 magnitude of a / S (ties to the even index, saturating at
 * 6) by exact comparison of a with S times the midpoints; the block error
 * err = ((e_0^2 + e_1^2) + e_2^2) + ... with e_i = a_i - m_i * S in float64,
 * no fused multiply-add (built with -ffp-contract=off); the least error wins,
 * the smallest code on equal errors. Pinned against the numpy version (and
 * through it against exact rational errors) by tests/test_oracle_nvfp4.py. */
#include <math.h>
#include <stdint.h>

static const double kMid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
static const double kMag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* value of a positive finite E4M3 code 1..126: 1 sign, 4 exponent (bias 7), 3 mantissa bits */
static double e4m3_value(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  if (e == 0) return ldexp((double)m / 8.0, -6);
  return ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* index 0..7 of the nearest E2M1 magnitude to a / S */
static int magnitude_index(double a, double S) {
  int idx = 0;
  for (int j = 0; j < 7; ++j) {
    const double t = S * kMid[j];
    if (a > t) idx++;
    else if (a == t && (j % 2 == 1)) idx++;  /* a tie between odd j and even j+1 goes up */
  }
  return idx;
}

double nvfp4_block_error(const double* a, double S) {
  double err = 0.0;
  for (int i = 0; i < 16; ++i) {
    const double e = a[i] - kMag[magnitude_index(a[i], S)] * S;
    err = err + e * e;
  }
  return err;
}

/* a: [nb][16] magnitudes; out: [nb] chosen codes 1..126 */
void nvfp4_choose_scales(const double* a, int64_t nb, double g, int32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    int best = 1;
    double best_err = 0.0;
    for (int c = 1; c <= 126; ++c) {
      const double err = nvfp4_block_error(a + 16 * b, e4m3_value(c) * g);
      if (c == 1 || err < best_err) {
        best = c;
        best_err = err;
      }
    }
    out[b] = best;
  }
}
