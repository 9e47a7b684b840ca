// ssm_oracle.cpp -- plain fp64 CPU reference of the selective state-space scan.
//
// TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
// checked against.  Only the test suite, the smoke check and the benchmark's
// CPU-baseline leg may load it.  It shares no code, header, table or helper
// with the GPU library, and the GPU library never calls it.
//
// What it computes is the plain definition of the method, evaluated one time
// step after another in double precision, with no blocking, chunking or
// reassociation:
//
//   * discrete recurrence h_k = Abar_k * h_{k-1} + Bbar_k * x_k and readout
//     y_k = C_k * h_k + D * x_k  (gsyq.cn "Mamba 状态空间模型深度解析", section
//     "连续到离散的转换", and the sequential loop in section "计算复杂度分析");
//     the same recurrence h_k = Abar h_{k-1} + Bbar x_k in the VMamba reading
//     note, section "循环结构表示以快速推理";
//   * Abar = exp(Delta * A) and the zero-order-hold input matrix
//     Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B (gsyq.cn, section
//     "连续到离散的转换"); for a diagonal A this is elementwise and Delta
//     cancels: Bbar[n] = (exp(Delta A[n]) - 1) / A[n] * B[n];
//   * the simplified input matrix Bbar = Delta * B used by the page's
//     parallel_scan sketch (gsyq.cn, section "硬件优化并行扫描算法");
//   * one independent single-input single-output SSM per channel d, with
//     A of shape (D, N), B and C of shape (batch, L, N) and Delta of shape
//     (batch, L, D) (VMamba note, section "mamba：从S4到S6的算法变化流程");
//     C is a 1 x N row, so the readout is a contraction over n (same note,
//     section "S4中三个矩阵的维度表示、维度变化");
//   * the skip term D * u added to the scan output, where u is the conv
//     output when the prologue is on (gsyq.cn SelectiveSSM.forward, which
//     returns the scan plus self.D * x_conv);
//   * the causal depthwise conv1d prologue, PyTorch Conv1d semantics with
//     padding K-1 keeping the first L outputs, followed by SiLU
//     silu(z) = z / (1 + exp(-z)) (gsyq.cn SelectiveSSM.__init__ / forward);
//   * optionally the step size is produced here from its pre-activation:
//     Delta = softplus(delta + bias[d]), softplus(v) = log(1 + exp(v)), the
//     bias being the per-channel bias of the Delta projection (gsyq.cn,
//     section "选择性的数学解析", Delta = Softplus(Linear(x)); VMamba note,
//     section "mamba：从S4到S6的算法变化流程", tau_Delta = softplus);
//   * optionally the output is gated by a second input stream z of the same
//     shape as x: out = y * silu(z) (the gated-MLP branch the Mamba block
//     adds around the SSM: VMamba note, section "简化的SSM架构"; the page's
//     figure with the formula is lost, so this is a reading);
//   * optionally the conv window continues across calls: conv_state_in holds
//     the K-1 inputs before token 0 (oldest first; zeros when absent) and
//     conv_state_out receives the last K-1 inputs, so a sequence scanned in
//     two calls, or a prefill followed by decode steps, sees the same window
//     as one call (the recurrent, constant-cost-per-token inference mode:
//     53ai.com explainer, section "一、Motivation").
//
// The backward pass (O3) is the reverse-mode derivative of the same
// sequential recurrence, written out with the chain rule and evaluated in
// fp64 from the last token to the first; the forward states it needs are
// kept from a plain forward sweep.  (The pages name training as the use of
// the parallel scan -- 53ai.com explainer, section "3.6 Empirical
// Evaluation" and VMamba note, section "硬件感知的设计" -- but print no
// gradient formula; the derivative of the defined function is the reading.)
//
// Readings where the pages are silent:
//   - the initial state h0 precedes token 0, so y_0 already contains x_0;
//   - Abar at step t uses Delta_t, the same step as x_t;
//   - with ZOH and A[d,n] == 0 the input factor is the limit Delta;
//   - decode (one token) updates the state first and reads y from the
//     updated state.
//
// Build: g++ -O2 -std=c++17 -shared -fPIC (no -ffast-math).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

struct ScanProblem {
  int64_t batch, seqlen, dim, dstate;
  const double *x, *delta, *delta_bias;
  int delta_softplus;
  const double *A, *Bm, *Cm, *Dskip, *z, *h0;
  const double *conv_w, *conv_b;
  int64_t conv_k;
  const double* conv_state_in;
  int zoh;
  double *y, *h_last, *conv_state_out;
};

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// softplus(v) = log(1 + exp(v)), written so that neither branch overflows.
double softplus(double v) { return (v > 0.0 ? v : 0.0) + std::log1p(std::exp(-std::fabs(v))); }

// The step size Delta[b, t, d]: the given value, plus the channel's bias when
// one is given, through softplus when asked.
double step_size(const ScanProblem& p, int64_t b, int64_t t, int64_t d) {
  double v = p.delta[(b * p.seqlen + t) * p.dim + d];
  if (p.delta_bias) v += p.delta_bias[d];
  return p.delta_softplus ? softplus(v) : v;
}

// x[b, t, d] for -(K-1) <= t < L: before token 0 the conv window holds
// conv_state_in[b, d, (K-1) + t] (zeros when no state is given).
double x_at(const ScanProblem& p, int64_t b, int64_t t, int64_t d) {
  if (t >= 0) return p.x[(b * p.seqlen + t) * p.dim + d];
  const int64_t S = p.conv_k - 1;
  if (!p.conv_state_in || t < -S) return 0.0;
  return p.conv_state_in[(b * p.dim + d) * S + S + t];
}

// Input factor multiplying B[n] * u: Delta (simplified) or the ZOH factor
// (exp(Delta A) - 1) / A, whose A -> 0 limit is Delta.
double input_factor(double dt, double a_cont, int zoh) {
  if (!zoh) return dt;
  if (a_cont == 0.0) return dt;
  return std::expm1(dt * a_cont) / a_cont;
}

// Scan input u[b, t, d]: x itself, or silu(bias + sum_k w[d,k] x[b, t-K+1+k, d])
// with x before the start of the sequence taken from the conv state.
double scan_input(const ScanProblem& p, int64_t b, int64_t t, int64_t d) {
  const int64_t L = p.seqlen, D = p.dim;
  if (!p.conv_w) return p.x[(b * L + t) * D + d];
  const int64_t K = p.conv_k;
  double z = p.conv_b ? p.conv_b[d] : 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t src = t - (K - 1) + k;
    z += p.conv_w[d * K + k] * x_at(p, b, src, d);
  }
  return silu(z);
}

// The sequential recurrence for one channel (b, d).
void scan_channel(const ScanProblem& p, int64_t b, int64_t d, std::vector<double>& h) {
  const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
  for (int64_t n = 0; n < N; ++n) h[n] = p.h0 ? p.h0[(b * D + d) * N + n] : 0.0;
  const double dskip = p.Dskip ? p.Dskip[d] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    const double u = scan_input(p, b, t, d);
    const double dt = step_size(p, b, t, d);
    const double* Bt = p.Bm + (b * L + t) * N;
    const double* Ct = p.Cm + (b * L + t) * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a_cont = p.A[d * N + n];
      const double abar = std::exp(dt * a_cont);
      const double bbar = input_factor(dt, a_cont, p.zoh) * Bt[n];
      h[n] = abar * h[n] + bbar * u;
      acc += Ct[n] * h[n];
    }
    double out = acc + dskip * u;
    if (p.z) out *= silu(p.z[(b * L + t) * D + d]);
    p.y[(b * L + t) * D + d] = out;
  }
  if (p.h_last)
    for (int64_t n = 0; n < N; ++n) p.h_last[(b * D + d) * N + n] = h[n];
  // the last K-1 inputs, oldest first (entry j reads conv_state_in only at
  // index j or above, so in ascending j the state may be updated in place)
  if (p.conv_w && p.conv_state_out) {
    const int64_t S = p.conv_k - 1;
    for (int64_t j = 0; j < S; ++j)
      p.conv_state_out[(b * D + d) * S + j] = x_at(p, b, L - S + j, d);
  }
}

void run_channels(const ScanProblem& p, int64_t first, int64_t last) {
  std::vector<double> h(p.dstate);
  for (int64_t c = first; c < last; ++c) scan_channel(p, c / p.dim, c % p.dim, h);
}

int pick_threads(int requested, int64_t work_items) {
  int n = requested > 0 ? requested : (int)std::thread::hardware_concurrency();
  if (n < 1) n = 1;
  if ((int64_t)n > work_items) n = (int)(work_items > 0 ? work_items : 1);
  return n;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

struct BwdProblem {
  int64_t batch, seqlen, dim, dstate;
  const double *x, *delta, *A, *Bm, *Cm, *Dskip, *h0, *dy, *dh_last;
  int zoh;
  double *dx, *ddelta, *dB, *dC, *dh0;   // dB, dC: rows of the batch rows a worker owns
  // Optional magnitudes (all NULL, or all given with the gradients' shapes):
  // for every gradient entry, the same chain-rule sum with every term, and
  // every quantity inside a term (states, adjoints, inputs), replaced by its
  // absolute value.  A sum evaluated in any order and precision with unit
  // roundoff u then differs from the exact one by at most about
  // (depth * u) times this magnitude (running error analysis), so a test can
  // bound each entry's error by a multiple of its own magnitude instead of
  // the largest entry of the tensor.
  double *mx, *mdelta, *mB, *mC, *mh0;
};

// d(input factor)/d(Delta) and d(input factor)/dA for the factor f used in
// Bbar = f * B: Delta*B has f = Delta (derivatives 1 and 0); ZOH has
// f = (exp(Delta A) - 1) / A, so df/dDelta = exp(Delta A) and
// df/dA = (Delta exp(Delta A) - f) / A, whose A -> 0 limit is Delta^2 / 2.
void factor_derivs(double dt, double a_cont, int zoh, double* df_dt, double* df_da) {
  if (!zoh) {
    *df_dt = 1.0;
    *df_da = 0.0;
    return;
  }
  if (a_cont == 0.0) {
    *df_dt = 1.0;
    *df_da = 0.5 * dt * dt;
    return;
  }
  const double e = std::exp(dt * a_cont);
  *df_dt = e;
  *df_da = (dt * e - std::expm1(dt * a_cont) / a_cont) / a_cont;
}

// Gradients for batch row b (all channels), accumulating dA (D, N) and
// dD (D) into the worker's own buffers.
void bwd_batch_row(const BwdProblem& p, int64_t b, std::vector<double>& dA,
                   std::vector<double>& dD, std::vector<double>& mA, std::vector<double>& mD) {
  const int64_t L = p.seqlen, D = p.dim, N = p.dstate;
  const bool mag = p.mx != nullptr;
  std::vector<double> H((L + 1) * N);   // H[(t + 1) * N + n] = h_t[n], row 0 = h_{-1}
  std::vector<double> g(N);
  // magnitudes of the states and adjoints (used only when `mag`)
  std::vector<double> Hm(mag ? (L + 1) * N : 0), gm(mag ? N : 0);
  for (int64_t d = 0; d < D; ++d) {
    // forward sweep keeping every state
    for (int64_t n = 0; n < N; ++n) H[n] = p.h0 ? p.h0[(b * D + d) * N + n] : 0.0;
    if (mag)
      for (int64_t n = 0; n < N; ++n) Hm[n] = std::fabs(H[n]);
    for (int64_t t = 0; t < L; ++t) {
      const double u = p.x[(b * L + t) * D + d];
      const double dt = p.delta[(b * L + t) * D + d];
      for (int64_t n = 0; n < N; ++n) {
        const double a_cont = p.A[d * N + n];
        const double abar = std::exp(dt * a_cont);
        const double inp = input_factor(dt, a_cont, p.zoh) * p.Bm[(b * L + t) * N + n] * u;
        H[(t + 1) * N + n] = abar * H[t * N + n] + inp;
        if (mag) Hm[(t + 1) * N + n] = abar * Hm[t * N + n] + std::fabs(inp);
      }
    }
    // reverse sweep: g[n] is dLoss/dh_t[n] once token t's output term is added
    for (int64_t n = 0; n < N; ++n) g[n] = p.dh_last ? p.dh_last[(b * D + d) * N + n] : 0.0;
    if (mag)
      for (int64_t n = 0; n < N; ++n) gm[n] = std::fabs(g[n]);
    const double dskip = p.Dskip ? p.Dskip[d] : 0.0;
    for (int64_t t = L - 1; t >= 0; --t) {
      const double u = p.x[(b * L + t) * D + d];
      const double dt = p.delta[(b * L + t) * D + d];
      const double gy = p.dy[(b * L + t) * D + d];
      double du = dskip * gy, ddt = 0.0;
      double mdu = std::fabs(dskip * gy), mddt = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double a_cont = p.A[d * N + n];
        const double Bn = p.Bm[(b * L + t) * N + n];
        const double Cn = p.Cm[(b * L + t) * N + n];
        const double h_prev = H[t * N + n];
        const double h_now = H[(t + 1) * N + n];
        const double G = g[n] + Cn * gy;                 // y_t = sum C h_t + ...
        const double abar = std::exp(dt * a_cont);
        const double f = input_factor(dt, a_cont, p.zoh);
        double df_dt, df_da;
        factor_derivs(dt, a_cont, p.zoh, &df_dt, &df_da);
        p.dC[(b * L + t) * N + n] += gy * h_now;
        p.dB[(b * L + t) * N + n] += G * f * u;
        du += G * f * Bn;
        // h_t = exp(dt A) h_{t-1} + f(dt, A) B u
        ddt += G * (a_cont * abar * h_prev + df_dt * Bn * u);
        dA[d * N + n] += G * (dt * abar * h_prev + df_da * Bn * u);
        g[n] = abar * G;                                  // into h_{t-1}
        if (mag) {
          const double Gm = gm[n] + std::fabs(Cn * gy);
          const double hpm = Hm[t * N + n], hnm = Hm[(t + 1) * N + n];
          p.mC[(b * L + t) * N + n] += std::fabs(gy) * hnm;
          p.mB[(b * L + t) * N + n] += Gm * std::fabs(f * u);
          mdu += Gm * std::fabs(f * Bn);
          mddt += Gm * (std::fabs(a_cont) * abar * hpm + std::fabs(df_dt * Bn * u));
          mA[d * N + n] += Gm * (std::fabs(dt) * abar * hpm + std::fabs(df_da * Bn * u));
          gm[n] = abar * Gm;
        }
      }
      p.dx[(b * L + t) * D + d] = du;
      p.ddelta[(b * L + t) * D + d] = ddt;
      dD[d] += gy * u;
      if (mag) {
        p.mx[(b * L + t) * D + d] = mdu;
        p.mdelta[(b * L + t) * D + d] = mddt;
        mD[d] += std::fabs(gy * u);
      }
    }
    if (p.dh0)
      for (int64_t n = 0; n < N; ++n) p.dh0[(b * D + d) * N + n] = g[n];
    if (mag)
      for (int64_t n = 0; n < N; ++n) p.mh0[(b * D + d) * N + n] = gm[n];
  }
}

}  // namespace

extern "C" {

// O1: y (batch, L, D) and optionally h_last (batch, D, N) from x, delta
// (batch, L, D), delta_bias (D) or NULL, A (D, N), B, C (batch, L, N), Dskip
// (D) or NULL, z (batch, L, D) or NULL, h0 (batch, D, N) or NULL, conv_w
// (D, K) / conv_b (D) or NULL, conv_state_in (batch, D, K-1) or NULL; writes
// conv_state_out (batch, D, K-1) when given with conv_w.  All arrays are
// row-major doubles.  Returns 0, or -1 on a bad argument.  Uses `nthreads`
// std::threads over the (b, d) channels (0 = all hardware threads).
int ssm_ref_scan_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                     const double* x, const double* delta, const double* delta_bias,
                     int delta_softplus, const double* A, const double* Bm,
                     const double* Cm, const double* Dskip, const double* z,
                     const double* h0, const double* conv_w, const double* conv_b,
                     int64_t conv_k, const double* conv_state_in, int zoh, double* y,
                     double* h_last, double* conv_state_out, int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return -1;
  if (conv_w && conv_k < 1) return -1;
  if (batch * dim == 0) return 0;
  if (seqlen > 0 && (!x || !delta || !Bm || !Cm || !y)) return -1;
  if (!A) return -1;
  ScanProblem p{batch, seqlen, dim, dstate, x, delta, delta_bias, delta_softplus, A, Bm,
                Cm, Dskip, z, h0, conv_w, conv_b, conv_k, conv_state_in, zoh, y, h_last,
                conv_state_out};
  const int64_t channels = batch * dim;
  const int nt = pick_threads(nthreads, channels);
  if (nt == 1) {
    run_channels(p, 0, channels);
    return 0;
  }
  std::vector<std::thread> pool;
  for (int i = 0; i < nt; ++i) {
    const int64_t first = channels * i / nt, last = channels * (i + 1) / nt;
    pool.emplace_back(run_channels, std::cref(p), first, last);
  }
  for (auto& th : pool) th.join();
  return 0;
}

// O2: one decode step.  h (batch, D, N) is read and overwritten with the new
// state; y (batch, D) = C . h_new + Dskip * u (times silu(z) when z is given).
// x, delta, z are (batch, D); B, C are (batch, N).  With conv_w the scan input
// u is the conv over the window conv_state (batch, D, K-1) followed by x, and
// conv_state is shifted in place to end with x.  This is O1 with L = 1.
int ssm_ref_step_f64(int64_t batch, int64_t dim, int64_t dstate, double* h,
                     const double* x, const double* delta, const double* delta_bias,
                     int delta_softplus, const double* A, const double* Bm,
                     const double* Cm, const double* Dskip, const double* z,
                     const double* conv_w, const double* conv_b, int64_t conv_k,
                     double* conv_state, int zoh, double* y, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1) return -1;
  if (conv_w && (conv_k < 1 || (conv_k > 1 && !conv_state))) return -1;
  if (batch * dim == 0) return 0;
  if (!h || !x || !delta || !A || !Bm || !Cm || !y) return -1;
  // h and conv_state are both input and output; the scan reads a channel's
  // inputs before it writes that channel's outputs, so in-place is safe.
  return ssm_ref_scan_f64(batch, 1, dim, dstate, x, delta, delta_bias, delta_softplus, A, Bm,
                          Cm, Dskip, z, h, conv_w, conv_b, conv_k, conv_state, zoh, y, h,
                          conv_state, nthreads);
}

// O3: gradients of the scalar loss sum(dy * y) + sum(dh_last * h_last) of
// O1 without conv prologue: dx, ddelta (batch, L, D), dA (D, N), dB, dC
// (batch, L, N), dD (D) and dh0 (batch, D, N) when their pointers are
// given.  dy is (batch, L, D); dh_last (batch, D, N) or NULL.  Outputs are
// overwritten.  Workers split the batch rows; dA and dD are summed over the
// workers in worker order.  Returns 0, or -1 on a bad argument.
int ssm_ref_scan_bwd_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         const double* x, const double* delta, const double* A,
                         const double* Bm, const double* Cm, const double* Dskip,
                         const double* h0, const double* dy, const double* dh_last, int zoh,
                         double* dx, double* ddelta, double* dA, double* dB, double* dC,
                         double* dD, double* dh0, int nthreads);

// O3 together with the magnitude of every gradient entry (see BwdProblem):
// mx, mdelta (batch, L, D), mA (D, N), mB, mC (batch, L, N), mD (D) and mh0
// (batch, D, N), all required.  The gradients are the same as
// ssm_ref_scan_bwd_f64's (dD and dh0 required here too).
int ssm_ref_scan_bwd_mag_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                             const double* x, const double* delta, const double* A,
                             const double* Bm, const double* Cm, const double* Dskip,
                             const double* h0, const double* dy, const double* dh_last,
                             int zoh, double* dx, double* ddelta, double* dA, double* dB,
                             double* dC, double* dD, double* dh0, double* mx, double* mdelta,
                             double* mA, double* mB, double* mC, double* mD, double* mh0,
                             int nthreads);

}  // extern "C"

namespace {

int scan_bwd_impl(const BwdProblem& p0, double* dA, double* dD, double* mA, double* mD,
                  int nthreads) {
  const int64_t batch = p0.batch, seqlen = p0.seqlen, dim = p0.dim, dstate = p0.dstate;
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return -1;
  if (!p0.A || !dA) return -1;
  if (batch * seqlen * dim > 0 && (!p0.x || !p0.delta || !p0.Bm || !p0.Cm || !p0.dy ||
                                   !p0.dx || !p0.ddelta || !p0.dB || !p0.dC))
    return -1;
  const bool mag = p0.mx != nullptr;
  const int64_t D = dim, N = dstate;
  for (int64_t i = 0; i < D * N; ++i) dA[i] = 0.0;
  if (dD)
    for (int64_t i = 0; i < D; ++i) dD[i] = 0.0;
  if (batch * seqlen > 0) {
    for (int64_t i = 0; i < batch * seqlen * N; ++i) p0.dB[i] = p0.dC[i] = 0.0;
  }
  if (mag) {
    for (int64_t i = 0; i < D * N; ++i) mA[i] = 0.0;
    for (int64_t i = 0; i < D; ++i) mD[i] = 0.0;
    for (int64_t i = 0; i < batch * seqlen * N; ++i) p0.mB[i] = p0.mC[i] = 0.0;
  }
  if (batch * dim == 0) return 0;
  const BwdProblem& p = p0;
  const int nt = pick_threads(nthreads, batch);
  std::vector<std::vector<double>> dA_w(nt, std::vector<double>(D * N, 0.0));
  std::vector<std::vector<double>> dD_w(nt, std::vector<double>(D, 0.0));
  std::vector<std::vector<double>> mA_w(nt, std::vector<double>(mag ? D * N : 0, 0.0));
  std::vector<std::vector<double>> mD_w(nt, std::vector<double>(mag ? D : 0, 0.0));
  auto work = [&](int w) {
    for (int64_t b = batch * w / nt; b < batch * (w + 1) / nt; ++b)
      bwd_batch_row(p, b, dA_w[w], dD_w[w], mA_w[w], mD_w[w]);
  };
  std::vector<std::thread> pool;
  for (int w = 1; w < nt; ++w) pool.emplace_back(work, w);
  work(0);
  for (auto& th : pool) th.join();
  for (int w = 0; w < nt; ++w) {
    for (int64_t i = 0; i < D * N; ++i) dA[i] += dA_w[w][i];
    if (dD)
      for (int64_t i = 0; i < D; ++i) dD[i] += dD_w[w][i];
    if (mag) {
      for (int64_t i = 0; i < D * N; ++i) mA[i] += mA_w[w][i];
      for (int64_t i = 0; i < D; ++i) mD[i] += mD_w[w][i];
    }
  }
  return 0;
}

}  // namespace

extern "C" {

int ssm_ref_scan_bwd_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                         const double* x, const double* delta, const double* A,
                         const double* Bm, const double* Cm, const double* Dskip,
                         const double* h0, const double* dy, const double* dh_last, int zoh,
                         double* dx, double* ddelta, double* dA, double* dB, double* dC,
                         double* dD, double* dh0, int nthreads) {
  const BwdProblem p{batch, seqlen, dim, dstate, x, delta, A, Bm, Cm, Dskip, h0, dy, dh_last,
                     zoh, dx, ddelta, dB, dC, dh0, nullptr, nullptr, nullptr, nullptr,
                     nullptr};
  return scan_bwd_impl(p, dA, dD, nullptr, nullptr, nthreads);
}

int ssm_ref_scan_bwd_mag_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                             const double* x, const double* delta, const double* A,
                             const double* Bm, const double* Cm, const double* Dskip,
                             const double* h0, const double* dy, const double* dh_last,
                             int zoh, double* dx, double* ddelta, double* dA, double* dB,
                             double* dC, double* dD, double* dh0, double* mx, double* mdelta,
                             double* mA, double* mB, double* mC, double* mD, double* mh0,
                             int nthreads) {
  if (!dD || !dh0 || !mx || !mdelta || !mA || !mB || !mC || !mD || !mh0) return -1;
  const BwdProblem p{batch, seqlen, dim, dstate, x, delta, A, Bm, Cm, Dskip, h0, dy, dh_last,
                     zoh, dx, ddelta, dB, dC, dh0, mx, mdelta, mB, mC, mh0};
  return scan_bwd_impl(p, dA, dD, mA, mD, nthreads);
}

}  // extern "C"
