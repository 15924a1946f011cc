/*
 * moe_oracle.c -- plain CPU oracle of the sparse Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU path never
 * calls it, links it or shares code with it.
 *
 * Every function is the plain definition of one step, written out with fp64
 * accumulation in ascending index order and compiled with -ffp-contract=off,
 * so that a reader can check it against the defining passage by eye:
 *
 *   logits      "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at
 *               Scale" -- Core claim (tokens are scored against experts and the
 *               top-K units are gathered per token).
 *   top-k       same page, Axiom ledger: the selection returns the *exact*
 *               global top-K indices.  Ties go to the lower expert id.
 *   gates       softmax over the k selected logits, so each token's weights sum
 *               to one.  The pages never name the normalisation; this is the
 *               plainest reading that keeps the weights a convex combination.
 *   counts/LIS  "A Replicate-and-Quantize Strategy for Plug-and-Play Load
 *               Balancing of Sparse Mixture-of-Experts LLMs" -- What carries the
 *               argument, and Definition 1 as quoted in its Circularity Check:
 *               n_j tokens routed to expert j, LIS = m * max_j n_j / (n * k).
 *   permutation OmniMoE -- What carries the argument and Figure 3: execution is
 *               inverted to expert-centric order, active experts compressed into
 *               contiguous groups.  Stable: within an expert, flat order t*k+j.
 *   expert FFN  "FloE: On-the-Fly MoE Inference on Memory-constrained GPU" --
 *               What carries the argument / Core claim / Figure 11: an expert is
 *               W_gate, W_up, W_down with SiLU applied to the gate projection and
 *               the up output feeding the down projection.
 *   shared      OmniMoE abstract and Figure 1: an always-active shared dense MLP
 *               branch next to the routed experts.
 *   INT4 decode "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient
 *               On-Device MoE-based LLM Serving" -- What carries the argument
 *               (asymmetric quantisation of the weight matrix), Assumptions &
 *               free parameters (group size 128), Figure 8 (dequantisation
 *               inside the GEMM kernel).
 *
 * Rounding points (the only choices, all fixed here):
 *   logits  : one rounding of the fp64 sum to fp32.
 *   gates   : one rounding of the fp64 softmax to fp32 (k = 1 gives 1 exactly).
 *   H       : rho() = one rounding of the fp64 activation to bf16 (bf16 layers)
 *             or to fp32 (fp32 layers), mirroring the stored intermediate.
 *   y       : one rounding of the fp64 weighted sum to fp32.
 *   INT4 W  : bf16_RNE( fp32( fp32(q) - fp32(z) ) * fp32(s) ), each fp32 op
 *             rounded to nearest even, no fused multiply-add.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NONFINITE 2

/* element types of input arrays */
#define ORC_F32 0
#define ORC_BF16 1

/* H rounding modes */
#define ORC_ROUND_NONE 0
#define ORC_ROUND_BF16 1
#define ORC_ROUND_F32 2

/* activations */
#define ORC_SWIGLU 0
#define ORC_RELU 1

/* ---- scalar conversions (exact) -------------------------------------- */

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static float fp16_to_float(uint16_t h) {
  /* IEEE binary16 -> binary32, exact for every input */
  uint32_t sign = (uint32_t)(h >> 15) & 1u;
  int exp = (h >> 10) & 0x1f;
  uint32_t man = h & 0x3ffu;
  float mag;
  if (exp == 0) {
    mag = ldexpf((float)man, -24); /* subnormal or zero */
  } else if (exp == 31) {
    mag = man ? NAN : INFINITY;
  } else {
    mag = ldexpf((float)(man | 0x400u), exp - 25);
  }
  return sign ? -mag : mag;
}

static double elem(const void* p, int dt, size_t i) {
  if (dt == ORC_BF16) return bf16_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

/* Round a double to the nearest bf16 value, ties to even (one rounding). */
double orc_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  (void)frexp(v, &e);      /* v = m * 2^e, 0.5 <= |m| < 1 */
  int q = e - 8;           /* quantum exponent for 8 significant bits */
  if (q < -133) q = -133;  /* bf16 subnormal quantum */
  double r = nearbyint(ldexp(v, -q)); /* default rounding mode: nearest-even */
  double out = ldexp(r, q);
  if (fabs(out) > 3.3895313892515355e38) return v > 0 ? INFINITY : -INFINITY;
  return out;
}

static double rho(double v, int mode) {
  if (mode == ORC_ROUND_BF16) return orc_round_bf16(v);
  if (mode == ORC_ROUND_F32) return (double)(float)v;
  return v;
}

/* ---- O1: router logits ------------------------------------------------ */
/* logits[t][e] = fp32( sum_i x[t][i] * W_r[e][i] + b[e] ), fp64 sum, i ascending. */
int orc_router_logits(const void* x, int xdt, const void* w_r, const float* b_r,
                      int T, int d, int E, float* logits) {
  if (T < 0 || d < 1 || E < 1 || !logits || (T > 0 && (!x || !w_r))) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int i = 0; i < d; ++i)
        s += elem(x, xdt, (size_t)t * d + i) * elem(w_r, xdt, (size_t)e * d + i);
      if (b_r) s += (double)b_r[e];
      logits[(size_t)t * E + e] = (float)s;
    }
  }
  return ORC_OK;
}

/* ---- O2/O3: exact top-k and softmax gates ----------------------------- */
/* Expert a precedes expert b iff l_a > l_b, or l_a == l_b and a < b (IEEE
 * comparison, so -0.0 == +0.0).  idx[t][0] is the largest.  Gates are the
 * softmax over the k selected logits, computed in fp64, rounded once. */
int orc_topk_gates(const float* logits, int T, int E, int k, int32_t* idx, float* gate) {
  if (T < 0 || E < 1 || k < 1 || k > E || (T > 0 && (!logits || !idx))) return ORC_ERR_ARG;
  for (size_t i = 0; i < (size_t)T * E; ++i)
    if (!isfinite(logits[i])) return ORC_ERR_NONFINITE;
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    int32_t* out = idx + (size_t)t * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        int taken = 0;
        for (int jj = 0; jj < j; ++jj) taken |= (out[jj] == e);
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower id on ties */
      }
      out[j] = best;
    }
    if (gate) {
      double m = (double)l[out[0]], sum = 0.0;
      for (int j = 0; j < k; ++j) sum += exp((double)l[out[j]] - m);
      for (int j = 0; j < k; ++j)
        gate[(size_t)t * k + j] = (float)(exp((double)l[out[j]] - m) / sum);
    }
  }
  return ORC_OK;
}

/* ---- O4..O7: counts, offsets, stable expert-major permutation, LIS ----- */
int orc_permute(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                int32_t* row_assign, int32_t* assign_row, double* lis) {
  if (T < 0 || E < 1 || k < 1 || k > E || !counts || !offsets) return ORC_ERR_ARG;
  size_t n = (size_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (size_t a = 0; a < n; ++a) {
    int e = idx[a];
    if (e < 0 || e >= E) return ORC_ERR_ARG;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!seen) return ORC_ERR_ARG;
  for (size_t a = 0; a < n; ++a) { /* ascending flat order a = t*k + j */
    int e = idx[a];
    int32_t row = offsets[e] + seen[e]++;
    if (row_assign) row_assign[row] = (int32_t)a;
    if (assign_row) assign_row[a] = row;
  }
  free(seen);
  if (lis) {
    int32_t mx = 0;
    for (int e = 0; e < E; ++e) if (counts[e] > mx) mx = counts[e];
    /* m = routed experts, n = tokens of this call, k = routed top-k */
    *lis = (T == 0) ? NAN : (double)((int64_t)E * mx) / (double)((int64_t)T * k);
  }
  return ORC_OK;
}

/* ---- Replica dispatch ---------------------------------------------------
 * "A Replicate-and-Quantize Strategy for Plug-and-Play Load Balancing of
 * Sparse Mixture-of-Experts LLMs" -- What carries the argument (a quantized
 * copy of the heaviest-loaded expert is appended to the layer) and the
 * review's If-this-is-right notes: the pages never fix how the unchanged
 * router's tokens reach the replica.  Reading taken here: the heavy expert's
 * assignments, in ascending flat order a = t*k + j, alternate between the
 * original (even rank 0, 2, ...) and the replica, which is expert slot E (odd
 * rank).  Counts, offsets, the permutation and LIS are then those of
 * orc_permute over E+1 slots (m = E+1 in the LIS). */
int orc_replica_split(const int32_t* idx, int T, int E, int k, int heavy, int32_t* idx_out) {
  if (T < 0 || E < 1 || k < 1 || k > E || heavy < 0 || heavy >= E || !idx_out) return ORC_ERR_ARG;
  size_t n = (size_t)T * k;
  int64_t rank = 0;
  for (size_t a = 0; a < n; ++a) {
    int e = idx[a];
    if (e < 0 || e >= E) return ORC_ERR_ARG;
    if (e == heavy) {
      idx_out[a] = (rank % 2 == 1) ? E : e;
      rank += 1;
    } else {
      idx_out[a] = e;
    }
  }
  return ORC_OK;
}

/* ---- O8/O9: expert FFN on (token, expert) pairs ------------------------ */
/* For pair p = (t, e):
 *   SwiGLU: H[f] = rho( silu(x_t . W_gate[e][f]) * (x_t . W_up[e][f]) ),
 *   ReLU  : H[f] = rho( max(0, x_t . W_in[e][f]) )  (W_in passed as w_up),
 *   Y[p][i] = sum_f H[f] * W_down[e][i][f]   (fp64, f ascending).
 * silu(v) = v / (1 + exp(-v)).  Weights of expert e start at e*F*d.
 * Y is returned in fp64 (no rounding). */
int orc_expert_rows(const void* x, int xdt, int d, int F, int act, const void* w_gate,
                    const void* w_up, const void* w_down, int wdt, int h_round,
                    const int32_t* tok, const int32_t* exp_id, int n, double* Y) {
  if (d < 1 || F < 1 || n < 0 || !x || !w_up || !w_down || !Y) return ORC_ERR_ARG;
  if (act == ORC_SWIGLU && !w_gate) return ORC_ERR_ARG;
  int err = 0;
#pragma omp parallel
  {
    double* h = (double*)malloc(sizeof(double) * (size_t)F);
    if (!h) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int p = 0; p < n; ++p) {
      if (!h) continue;
      size_t t = (size_t)tok[p], e = (size_t)exp_id[p];
      size_t xo = t * (size_t)d;
      for (int f = 0; f < F; ++f) {
        size_t wo = (e * (size_t)F + (size_t)f) * (size_t)d;
        double u = 0.0;
        for (int i = 0; i < d; ++i) u += elem(x, xdt, xo + i) * elem(w_up, wdt, wo + i);
        double v;
        if (act == ORC_SWIGLU) {
          double g = 0.0;
          for (int i = 0; i < d; ++i) g += elem(x, xdt, xo + i) * elem(w_gate, wdt, wo + i);
          v = (g / (1.0 + exp(-g))) * u;
        } else {
          v = u > 0.0 ? u : 0.0;
        }
        h[f] = rho(v, h_round);
      }
      for (int i = 0; i < d; ++i) {
        size_t wo = (e * (size_t)d + (size_t)i) * (size_t)F;
        double s = 0.0;
        for (int f = 0; f < F; ++f) s += h[f] * elem(w_down, wdt, wo + f);
        Y[(size_t)p * d + i] = s;
      }
    }
    free(h);
  }
  return err ? ORC_ERR_ARG : ORC_OK;
}

/* ---- O10: weighted combine back to token order ------------------------ */
/* y[t][i] = fp32( sum_{j<k} gate[t][j] * Y[assign_row[t*k+j]][i] + Ys[t][i] ),
 * j ascending in slot order, then the shared-expert term.  Y is indexed by
 * expert-major row; assign_row NULL means Y is already in flat (t*k+j) order.
 * Ys (shared experts) may be NULL. */
int orc_combine(const double* Y, const int32_t* assign_row, const float* gate, const double* Ys,
                int T, int k, int d, float* y) {
  if (T < 0 || k < 1 || d < 1 || (T > 0 && (!Y || !gate || !y))) return ORC_ERR_ARG;
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < d; ++i) {
      double s = 0.0;
      for (int j = 0; j < k; ++j) {
        size_t a = (size_t)t * k + j;
        size_t r = assign_row ? (size_t)assign_row[a] : a;
        s += (double)gate[a] * Y[r * d + i];
      }
      if (Ys) s += Ys[(size_t)t * d + i];
      y[(size_t)t * d + i] = (float)s;
    }
  return ORC_OK;
}

/* ---- O11: asymmetric group-wise INT4 decode --------------------------- */
/* q: [rows][K/8] int32, nibble i of word j is K-index 8j+i (low nibble first).
 * scale, zero: fp16 bits [rows][K/group].  Output: bf16 bits [rows][K]. */
int orc_dequant_int4(const int32_t* q, const uint16_t* scale, const uint16_t* zero,
                     int64_t rows, int K, int group, uint16_t* out) {
  if (rows < 0 || K < 8 || K % 8 || group < 8 || K % group || !q || !scale || !zero || !out)
    return ORC_ERR_ARG;
  int ng = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int kk = 0; kk < K; ++kk) {
      uint32_t word = (uint32_t)q[r * (K / 8) + kk / 8];
      uint32_t nib = (word >> (4 * (kk % 8))) & 0xFu;
      float s = fp16_to_float(scale[r * ng + kk / group]);
      float z = fp16_to_float(zero[r * ng + kk / group]);
      float a = (float)nib - z; /* one fp32 rounding */
      float b = a * s;          /* one fp32 rounding */
      double w = orc_round_bf16((double)b);
      float wf = (float)w;
      uint32_t u;
      memcpy(&u, &wf, 4);
      out[r * K + kk] = (uint16_t)(u >> 16);
    }
  }
  return ORC_OK;
}

/* ---- Nested (matryoshka) weight decode -------------------------------------
 * "D^2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device
 * MoE-based LLM Serving" -- What carries the argument: the lowest bit width is
 * an asymmetric quantisation of the weights, and every higher bit width adds a
 * binary residual of the remaining error, so INT2 sits inside INT3 inside INT4;
 * Assumptions & free parameters: group size 128.  Readings fixed here (the
 * pages give no formula): the residual of width b is one bit r_b per weight and
 * one fp16 magnitude a_b per group, adding +a_b (r_b = 1) or -a_b (r_b = 0).
 *   q2 : [rows][K/16] int32; word j holds K-indices 16j..16j+15, byte-transposed:
 *        K-index 16j + 4m + b sits in 2-bit field 4b + m (bits 8b+2m, 8b+2m+1);
 *   s2, z2 : fp16 [rows][K/group]  (base scale and zero point)
 *   p3, p4 : [rows][K/32] int32; word j holds K-indices 32j..32j+31, K-index
 *        32j + 4i + b in bit 8b + i (b < 4, i < 8);
 *   a3, a4 : fp16 [rows][K/group]  (residual magnitudes)
 * Decoded at width `bits` (2, 3 or 4), each fp32 operation rounded to nearest
 * even, no fused multiply-add, one bf16 rounding at the end:
 *   w = fp32( fp32(q2) - z2 ) * s2 ;  bits >= 3: w = w + (r3 ? a3 : -a3) ;
 *   bits == 4: w = w + (r4 ? a4 : -a4) ;  out = bf16_RNE(w). */
/* field of a 2-bit code and bit of a residual inside their storage words */
static int mwq_field(int kk) {
  int i = kk % 16;
  return 4 * (i % 4) + i / 4;
}
static int mwq_bit(int kk) {
  int i = kk % 32;
  return 8 * (i % 4) + i / 4;
}
int orc_dequant_mwq(const int32_t* q2, const uint16_t* s2, const uint16_t* z2, const int32_t* p3,
                    const uint16_t* a3, const int32_t* p4, const uint16_t* a4, int64_t rows,
                    int K, int group, int bits, uint16_t* out) {
  if (rows < 0 || K < 32 || K % 32 || group < 32 || K % group || !q2 || !s2 || !z2 || !out ||
      bits < 2 || bits > 4 || (bits >= 3 && (!p3 || !a3)) || (bits == 4 && (!p4 || !a4)))
    return ORC_ERR_ARG;
  int ng = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int kk = 0; kk < K; ++kk) {
      size_t g = (size_t)r * ng + kk / group;
      uint32_t w2 = (uint32_t)q2[r * (K / 16) + kk / 16];
      uint32_t q = (w2 >> (2 * mwq_field(kk))) & 0x3u;
      float s = fp16_to_float(s2[g]);
      float z = fp16_to_float(z2[g]);
      float a = (float)q - z; /* one fp32 rounding */
      float w = a * s;        /* one fp32 rounding */
      if (bits >= 3) {
        uint32_t bit = ((uint32_t)p3[r * (K / 32) + kk / 32] >> mwq_bit(kk)) & 1u;
        float m = fp16_to_float(a3[g]);
        w = w + (bit ? m : -m);
      }
      if (bits == 4) {
        uint32_t bit = ((uint32_t)p4[r * (K / 32) + kk / 32] >> mwq_bit(kk)) & 1u;
        float m = fp16_to_float(a4[g]);
        w = w + (bit ? m : -m);
      }
      double wr = orc_round_bf16((double)w);
      float wf = (float)wr;
      uint32_t u;
      memcpy(&u, &wf, 4);
      out[r * K + kk] = (uint16_t)(u >> 16);
    }
  }
  return ORC_OK;
}

/* ---- Contextual sparse down-projection ------------------------------------
 * "FloE: On-the-Fly MoE Inference on Memory-constrained GPU" -- Core claim and
 * What carries the argument: a channel of the expert's hidden layer whose
 * up-projection output is small in magnitude is pruned, which removes its gate
 * row and its down-projection column from the work; the up projection itself
 * is kept (quantised to INT2).  Assumptions & free parameters: one threshold per
 * expert, read off the empirical distribution of calibration activations.
 * Per (token, expert) row p, all in fp64 unless stated:
 *   u_f    = x_t . W_up[e][f]             (W_up: the decoded INT2 weights, bf16)
 *   keep_f = |u_f| > thr[e]               (decided on u_given[p][f] when given)
 *   h_f    = keep_f ? bf16_RNE( silu(x_t . W_gate[e][f]) * u_f ) : 0
 *   Y[p]   = W_down[e] . h
 * x [T][d], w_gate / w_up [E][F][d], w_down [E][d][F]: bf16 bits.  u_out
 * [n][F] and keep_out [n][F] may be NULL. */
int orc_floe_rows(const uint16_t* x, int d, int F, const uint16_t* w_gate, const uint16_t* w_up,
                  const uint16_t* w_down, const float* thr, const int32_t* tok,
                  const int32_t* exp_id, int n, const float* u_given, double* u_out,
                  uint8_t* keep_out, double* Y) {
  if (d < 1 || F < 1 || n < 0 || !x || !w_gate || !w_up || !w_down || !thr || !Y)
    return ORC_ERR_ARG;
  int err = 0;
#pragma omp parallel
  {
    double* h = (double*)malloc(sizeof(double) * (size_t)F);
    if (!h) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int p = 0; p < n; ++p) {
      if (!h) continue;
      size_t t = (size_t)tok[p], e = (size_t)exp_id[p];
      size_t xo = t * (size_t)d;
      for (int f = 0; f < F; ++f) {
        size_t wo = (e * (size_t)F + (size_t)f) * (size_t)d;
        double u = 0.0;
        for (int i = 0; i < d; ++i) u += bf16_to_double(x[xo + i]) * bf16_to_double(w_up[wo + i]);
        double mag = u_given ? fabs((double)u_given[(size_t)p * F + f]) : fabs(u);
        int keep = mag > (double)thr[e];
        if (u_out) u_out[(size_t)p * F + f] = u;
        if (keep_out) keep_out[(size_t)p * F + f] = (uint8_t)keep;
        if (keep) {
          double g = 0.0;
          for (int i = 0; i < d; ++i)
            g += bf16_to_double(x[xo + i]) * bf16_to_double(w_gate[wo + i]);
          h[f] = orc_round_bf16((g / (1.0 + exp(-g))) * u);
        } else {
          h[f] = 0.0;
        }
      }
      for (int i = 0; i < d; ++i) {
        size_t wo = (e * (size_t)d + (size_t)i) * (size_t)F;
        double s = 0.0;
        for (int f = 0; f < F; ++f) s += h[f] * bf16_to_double(w_down[wo + f]);
        Y[(size_t)p * d + i] = s;
      }
    }
    free(h);
  }
  return err ? ORC_ERR_ARG : ORC_OK;
}

/* ---- Atomic experts on a Cartesian router grid ------------------------------
 * "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale" -- What
 * carries the argument and Core claim: an atomic expert is one vector pair
 * (w_in, w_out) with output act(x . w_in) w_out (Eq. 4); the router treats an
 * expert id as a cell (i, j) of an Nr x Nc grid and scores it as the sum of a
 * row and a column log-probability (Eq. 8); each token assembles its top-K
 * atomic experts (Dynamic Expert Assembly). */

/* Row-wise log-softmax of an [T][n] fp32 matrix: fp64 inside, rounded once. */
int orc_log_softmax_rows(const float* l, int T, int n, float* out) {
  if (T < 0 || n < 1 || (T > 0 && (!l || !out))) return ORC_ERR_ARG;
  for (int t = 0; t < T; ++t) {
    const float* r = l + (size_t)t * n;
    double m = r[0];
    for (int i = 1; i < n; ++i) if (r[i] > m) m = r[i];
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += exp((double)r[i] - m);
    double lse = m + log(s);
    for (int i = 0; i < n; ++i) out[(size_t)t * n + i] = (float)((double)r[i] - lse);
  }
  return ORC_OK;
}

typedef struct {
  float s;
  int32_t id;
} orc_scored;

static int cmp_scored(const void* a, const void* b) {
  const orc_scored* x = (const orc_scored*)a;
  const orc_scored* y = (const orc_scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int cmp_int32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Exact top-K over the grid S_ij = fp32(pr[t][i] + pc[t][j]), expert id
 * n = i*Nc + j: (i,j) precedes (i',j') iff S > S', or S == S' and n < n'.  The
 * K chosen ids of a token are written in ascending id order (the slot order);
 * gates are the softmax over their S, fp64 inside (sum in slot order), rounded
 * once. */
int orc_grid_topk(const float* pr, const float* pc, int T, int Nr, int Nc, int K, int32_t* idx,
                  float* gate) {
  if (T < 0 || Nr < 1 || Nc < 1 || K < 1 || (int64_t)K > (int64_t)Nr * Nc || !idx || !gate)
    return ORC_ERR_ARG;
  const int N = Nr * Nc;
  int err = 0;
#pragma omp parallel
  {
    orc_scored* sc = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)N);
    double* w = (double*)malloc(sizeof(double) * (size_t)K);
    if (!sc || !w) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
      if (!sc || !w) continue;
      for (int i = 0; i < Nr; ++i)
        for (int j = 0; j < Nc; ++j) {
          float s = pr[(size_t)t * Nr + i] + pc[(size_t)t * Nc + j];
          sc[i * Nc + j].s = s;
          sc[i * Nc + j].id = i * Nc + j;
        }
      qsort(sc, (size_t)N, sizeof(orc_scored), cmp_scored);
      int32_t* out = idx + (size_t)t * K;
      double m = (double)sc[0].s;
      for (int s = 0; s < K; ++s) out[s] = sc[s].id;
      qsort(out, (size_t)K, sizeof(int32_t), cmp_int32);
      double sum = 0.0;
      for (int s = 0; s < K; ++s) {
        int n = out[s];
        float sv = pr[(size_t)t * Nr + n / Nc] + pc[(size_t)t * Nc + n % Nc];
        w[s] = exp((double)sv - m);
        sum += w[s];
      }
      for (int s = 0; s < K; ++s) gate[(size_t)t * K + s] = (float)(w[s] / sum);
    }
    free(sc);
    free(w);
  }
  return err ? ORC_ERR_ARG : ORC_OK;
}

/* Atomic-expert rows, per token p of the list (t = tok[p]):
 *   Y[p] = sum over slots s (ascending) of w_out[:, n_s] * bf16_RNE(g_s * act(x_t . w_in[n_s]))
 * fp64 accumulation; act 0 = SiLU, 1 = ReLU.  x [T][d], w_in [N][d], w_out
 * [d][N] (bf16 bits), idx/gate [T][K]. */
int orc_atomic_rows(const uint16_t* x, int d, const uint16_t* w_in, const uint16_t* w_out, int N,
                    const int32_t* idx, const float* gate, int K, int act, const int32_t* tok,
                    int n, double* Y) {
  if (d < 1 || N < 1 || K < 1 || n < 0 || !x || !w_in || !w_out || !idx || !gate || !Y)
    return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int p = 0; p < n; ++p) {
    size_t t = (size_t)tok[p];
    double* y = Y + (size_t)p * d;
    for (int i = 0; i < d; ++i) y[i] = 0.0;
    for (int s = 0; s < K; ++s) {
      size_t e = (size_t)idx[t * K + s];
      double u = 0.0;
      for (int i = 0; i < d; ++i)
        u += bf16_to_double(x[t * d + i]) * bf16_to_double(w_in[e * d + i]);
      double h = act == 0 ? u / (1.0 + exp(-u)) : (u > 0.0 ? u : 0.0);
      double a = orc_round_bf16((double)gate[t * K + s] * h);
      for (int i = 0; i < d; ++i) y[i] += a * bf16_to_double(w_out[(size_t)i * N + e]);
    }
  }
  return ORC_OK;
}
