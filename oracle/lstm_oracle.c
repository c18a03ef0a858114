/*
 * lstm_oracle.c -- plain fp64 CPU oracle for a single-layer, unidirectional
 * LSTM: forward pass and backpropagation through time.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test-suite, the smoke check and the CPU-baseline leg of the benchmark
 * load it.  It shares no header, helper, constant or table with the HIP
 * library; the gate and column order below are restated here from the
 * equations, on purpose, not included from the library's header.
 *
 * What it computes follows the "SingleLayerLstmGrad" operator page of the
 * Ascend CANN ops-nn repository:
 *   - forward: the table "前向传播公式" (input concatenation z_t=[h_{t-1};x_t],
 *     forget/input/output gates sigma(W z + b), candidate tanh(W z + b),
 *     c_t = f.c_{t-1} + i.g, h_t = o.tanh(c_t));
 *   - backward: "反向传播算法" steps 1-6 (current hidden gradient, cell
 *     gradient, the four gate deltas, parameter gradient sums, propagation
 *     to the previous step through W^T, and the carries), with the cell
 *     gradient derivation of "梯度计算原理" deciding how the forget gate enters
 *     the cell carry (it is applied once, see below).
 *
 * Conventions (readings of the page, each stated where it is used):
 *   - time is 0-based, t = 0..T-1, with h_{-1} = h0 and c_{-1} = c0 (the
 *     parameter table defines inith/initc as the state "at t=0 of h(t-1)");
 *   - W is [4H, H+I], row-major; row block k (rows [kH,(k+1)H)) is gate
 *     k in the order i, f, g, o ("ifjo", j being the candidate g); columns
 *     [0,H) multiply h_{t-1} and [H,H+I) multiply x_t, the order of z_t;
 *   - one bias b[4H] in the same gate order (NULL means zero);
 *   - all tensors are time-major: x [T,B,I], y [T,B,H], gates [T,B,4H];
 *   - the backward receives dy [T,B,H] (gradient of every output h_t), and
 *     optional dhT/dcT [B,H] (gradient of the final h and c), NULL = zero.
 *     The gradient of the last hidden state adds to dy_{T-1};
 *   - every gate delta is taken with respect to the gate's pre-activation
 *     (the forget-gate derivation on the page says so explicitly).
 *
 * Summation order is fixed (k ascending inside every dot product; t
 * descending then b ascending in the parameter-gradient sums), so the result
 * does not depend on the number of OpenMP threads.  No -ffast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sigm(double u) { return 1.0 / (1.0 + exp(-u)); }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* n > 0: that many OpenMP threads; n <= 0: one per available processor */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
#else
  (void)n;
#endif
}

/*
 * Forward pass ("前向传播公式" table).
 *   reverse: 0, or 1 for the reverse direction of the operator's direction
 *            attribute ("参数说明"): the steps run from t = T-1 down to 0, so
 *            the step at time t reads the state of time t+1 and h0/c0 enter
 *            at t = T-1; hT/cT are the state after the step at t = 0.
 *   x  [T,B,I], W [4H,H+I], b [4H] or NULL, h0/c0 [B,H] or NULL (zero state)
 *   mask [T,B,H] or NULL (all ones): the seq_length input of the parameter
 *            table ("参数说明"), a mask matrix standing for the actual length
 *            of each sequence.  Reading: the step's new cell and hidden
 *            values are blended with the state it read, element by element,
 *            c_t = m*c_new + (1-m)*c_{t-1} and h_t = m*h_new + (1-m)*h_{t-1},
 *            so that a step with m = 0 leaves the state as it was (padding
 *            past a sequence's end changes neither state nor gradient) and
 *            m = 1 is the plain cell; y_t is the state h_t
 *   y  [T,B,H]      h_t for every step (the layer output)
 *   hT, cT [B,H]    state after the last step (may be NULL)
 *   gates [T,B,4H]  activated gates i,f,g,o per step (kept for the backward;
 *                   may be NULL only if the caller will not run the backward)
 *   cell  [T,B,H]   c_t per step (same remark)
 * Returns 0, or -1 on a bad size / allocation failure.
 */
int oracle_lstm_fwd(long T, long B, long I, long H, int reverse,
                    const double* x, const double* W, const double* b,
                    const double* h0, const double* c0, const double* mask,
                    double* y, double* hT, double* cT,
                    double* gates, double* cell) {
  if (T < 0 || B < 0 || I < 0 || H <= 0) return -1;
  const long Z = H + I, G4 = 4 * H;
  double* hp = (double*)calloc((size_t)(B * H) + 1, sizeof(double)); /* h_{t-1} */
  double* cp = (double*)calloc((size_t)(B * H) + 1, sizeof(double)); /* c_{t-1} */
  double* a = (double*)malloc(((size_t)(B * G4) + 1) * sizeof(double));
  if (!hp || !cp || !a) { free(hp); free(cp); free(a); return -1; }
  if (h0) memcpy(hp, h0, (size_t)(B * H) * sizeof(double));
  if (c0) memcpy(cp, c0, (size_t)(B * H) * sizeof(double));

  for (long s = 0; s < T; ++s) {
    const long t = reverse ? T - 1 - s : s; /* time of the s-th step */
    const double* xt = x + t * B * I;
    /* pre-activation a = W z_t + b with z_t = [h_{t-1}; x_t] */
#pragma omp parallel for schedule(static)
    for (long br = 0; br < B * G4; ++br) {
      const long bb = br / G4, r = br % G4;
      const double* wr = W + r * Z;
      double s = b ? b[r] : 0.0;
      for (long k = 0; k < H; ++k) s += wr[k] * hp[bb * H + k];
      for (long k = 0; k < I; ++k) s += wr[H + k] * xt[bb * I + k];
      a[br] = s;
    }
    /* gates, cell and hidden state; (b, j) elements are independent, so
       h_{t-1}/c_{t-1} of (b, j) can be replaced in place by h_t/c_t */
    for (long bb = 0; bb < B; ++bb) {
      for (long j = 0; j < H; ++j) {
        const double* ab = a + bb * G4;
        const double ig = sigm(ab[j]);          /* input gate      */
        const double fg = sigm(ab[H + j]);      /* forget gate     */
        const double gg = tanh(ab[2 * H + j]);  /* candidate state */
        const double og = sigm(ab[3 * H + j]);  /* output gate     */
        const long o = t * B + bb;
        const double m = mask ? mask[o * H + j] : 1.0;
        const double cn = fg * cp[bb * H + j] + ig * gg; /* new cell value     */
        const double hn = og * tanh(cn);                 /* new hidden value   */
        const double c = m * cn + (1.0 - m) * cp[bb * H + j];
        const double h = m * hn + (1.0 - m) * hp[bb * H + j];
        if (gates) {
          gates[o * G4 + j] = ig;
          gates[o * G4 + H + j] = fg;
          gates[o * G4 + 2 * H + j] = gg;
          gates[o * G4 + 3 * H + j] = og;
        }
        if (cell) cell[o * H + j] = c;
        y[o * H + j] = h;
        hp[bb * H + j] = h;
        cp[bb * H + j] = c;
      }
    }
  }
  if (hT) memcpy(hT, hp, (size_t)(B * H) * sizeof(double));
  if (cT) memcpy(cT, cp, (size_t)(B * H) * sizeof(double));
  free(hp); free(cp); free(a);
  return 0;
}

/*
 * Backward pass ("反向传播算法" steps 1-6) from the stored forward values.
 *   reverse as in the forward (the recursion then runs from t = 0 up to T-1:
 *   the reverse of the forward's step order, whichever the direction);
 *   x, W, h0, c0, mask as in the forward; y, gates, cell as the forward
 *   wrote them;
 *   dy [T,B,H]; dhT, dcT [B,H] or NULL (zero).
 * Outputs (overwritten, never accumulated into):
 *   dx [T,B,I], dW [4H,H+I], db [4H] (may be NULL), dh0, dc0 [B,H]
 *   dgates [T,B,4H] optional: the gate deltas (i,f,g,o blocks) per step
 *   dcell  [T,B,H]  optional: the cell gradient delta-c_t of step 2 per step
 *
 * Carries.  Step 2 of the page adds "delta-c_next . f_next" while step 5
 * already defines the carry delta-c_prev = delta-c_t . f_t and step 6 hands
 * that product on as delta-c_next; taken literally f would be applied twice.
 * The derivation "细胞状态梯度推导" (d c_{t+1} / d c_t = f_{t+1}) fixes the
 * meaning: the forget factor enters once, so the carry delta-c_prev (which
 * already holds the factor) is added as it is.  The carries start from the
 * given final-state gradients: delta-h = dhT, delta-c = dcT.
 *
 * Mask (the blend of the forward): with m the step's mask value, the new
 * hidden and cell values receive m times the step's gradients, and the
 * state the step read receives the other (1-m) part directly --
 *   delta-h_new = m.delta-h,  delta-c_new = m.delta-c + delta-h_new.o.(1-tanh^2 c_new),
 *   carries: delta-c_prev = (1-m).delta-c + delta-c_new.f,
 *            delta-h_prev = (1-m).delta-h + (W^T delta-gates)[0,H);
 * the gate deltas are those of steps 2-3 with delta-h_new, delta-c_new in
 * place of delta-h, delta-c.  c_new = f.c_{t-1} + i.g is formed again from
 * the stored gates and the stored cell state of the previous step (the same
 * expression on the same values as in the forward).  With m = 1 this is the
 * page's recursion unchanged.
 */
int oracle_lstm_bwd(long T, long B, long I, long H, int reverse,
                    const double* x, const double* W,
                    const double* h0, const double* c0, const double* mask,
                    const double* y, const double* gates, const double* cell,
                    const double* dy, const double* dhT, const double* dcT,
                    double* dx, double* dW, double* db,
                    double* dh0, double* dc0,
                    double* dgates, double* dcell) {
  if (T < 0 || B < 0 || I < 0 || H <= 0) return -1;
  const long Z = H + I, G4 = 4 * H;
  double* dhc = (double*)calloc((size_t)(B * H) + 1, sizeof(double)); /* delta-h carry */
  double* dcc = (double*)calloc((size_t)(B * H) + 1, sizeof(double)); /* delta-c carry */
  double* dhp = (double*)calloc((size_t)(B * H) + 1, sizeof(double)); /* (1-m).delta-h of the step */
  double* dG = dgates;
  int own_dG = 0;
  if (!dG) {
    dG = (double*)malloc(((size_t)(T * B * G4) + 1) * sizeof(double));
    own_dG = 1;
  }
  if (!dhc || !dcc || !dhp || !dG) {
    free(dhc); free(dcc); free(dhp); if (own_dG) free(dG);
    return -1;
  }
  if (dhT) memcpy(dhc, dhT, (size_t)(B * H) * sizeof(double));
  if (dcT) memcpy(dcc, dcT, (size_t)(B * H) * sizeof(double));

  for (long s = T - 1; s >= 0; --s) {
    const long t = reverse ? T - 1 - s : s; /* time of the s-th forward step */
    /* steps 1-3 and the cell carry of step 5 (elementwise per (b, j)) */
    for (long bb = 0; bb < B; ++bb) {
      for (long j = 0; j < H; ++j) {
        const long o = t * B + bb;
        const double ig = gates[o * G4 + j];
        const double fg = gates[o * G4 + H + j];
        const double gg = gates[o * G4 + 2 * H + j];
        const double og = gates[o * G4 + 3 * H + j];
        const double c = cell[o * H + j];
        double cprev = t > 0 ? cell[(o - B) * H + j] : (c0 ? c0[bb * H + j] : 0.0);
        if (reverse) cprev = t < T - 1 ? cell[(o + B) * H + j] : (c0 ? c0[bb * H + j] : 0.0);
        const double m = mask ? mask[o * H + j] : 1.0;
        const double cn = mask ? fg * cprev + ig * gg : c;             /* the step's new cell value */
        const double tc = tanh(cn);
        const double dh = dy[o * H + j] + dhc[bb * H + j];             /* step 1 */
        const double dhn = m * dh;
        const double dc = dhn * og * (1.0 - tc * tc) + m * dcc[bb * H + j]; /* step 2 */
        const double d_o = dhn * tc * og * (1.0 - og);                 /* step 3 */
        const double d_g = dc * ig * (1.0 - gg * gg);
        const double d_i = dc * gg * ig * (1.0 - ig);
        const double d_f = dc * cprev * fg * (1.0 - fg);
        dG[o * G4 + j] = d_i;
        dG[o * G4 + H + j] = d_f;
        dG[o * G4 + 2 * H + j] = d_g;
        dG[o * G4 + 3 * H + j] = d_o;
        if (dcell) dcell[o * H + j] = dc;
        dcc[bb * H + j] = (1.0 - m) * dcc[bb * H + j] + dc * fg;       /* step 5: delta-c_prev */
        dhp[bb * H + j] = (1.0 - m) * dh;                              /* the state's own part */
      }
    }
    /* step 5: delta-z = W^T delta-gates; the first H entries go to the
       previous hidden state, the remaining I entries are the input gradient */
#pragma omp parallel for schedule(static)
    for (long bk = 0; bk < B * Z; ++bk) {
      const long bb = bk / Z, k = bk % Z;
      const double* g = dG + (t * B + bb) * G4;
      double s = 0.0;
      for (long r = 0; r < G4; ++r) s += W[r * Z + k] * g[r];
      if (k < H) dhc[bb * H + k] = dhp[bb * H + k] + s; /* step 6: delta-h_next */
      else dx[(t * B + bb) * I + (k - H)] = s;
    }
  }

  /* step 4: dW = sum_t delta-gates_t z_t^T, db = sum_t delta-gates_t,
     each element summed over t descending, then b ascending */
#pragma omp parallel for schedule(static)
  for (long r = 0; r < G4; ++r) {
    double* dwr = dW + r * Z;
    for (long k = 0; k < Z; ++k) dwr[k] = 0.0;
    double sb = 0.0;
    for (long t = T - 1; t >= 0; --t) {
      for (long bb = 0; bb < B; ++bb) {
        const double g = dG[(t * B + bb) * G4 + r];
        const double* hprev = t > 0 ? y + ((t - 1) * B + bb) * H : (h0 ? h0 + bb * H : NULL);
        if (reverse) hprev = t < T - 1 ? y + ((t + 1) * B + bb) * H : (h0 ? h0 + bb * H : NULL);
        const double* xt = x + (t * B + bb) * I;
        for (long k = 0; k < H; ++k) dwr[k] += g * (hprev ? hprev[k] : 0.0);
        for (long k = 0; k < I; ++k) dwr[H + k] += g * xt[k];
        sb += g;
      }
    }
    if (db) db[r] = sb;
  }

  if (dh0) memcpy(dh0, dhc, (size_t)(B * H) * sizeof(double));
  if (dc0) memcpy(dc0, dcc, (size_t)(B * H) * sizeof(double));
  free(dhc); free(dcc); free(dhp);
  if (own_dG) free(dG);
  return 0;
}
