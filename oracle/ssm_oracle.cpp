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
//     silu(z) = z / (1 + exp(-z)) (gsyq.cn SelectiveSSM.__init__ / forward).
//
// Readings where the pages are silent (listed in the design notes too):
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
  const double *x, *delta, *A, *Bm, *Cm, *Dskip, *h0;
  const double *conv_w, *conv_b;
  int64_t conv_k;
  int zoh;
  double *y, *h_last;
};

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// Input factor multiplying B[n] * u: Delta (simplified) or the ZOH factor
// (exp(Delta A) - 1) / A, whose A -> 0 limit is Delta.
double input_factor(double dt, double a_cont, int zoh) {
  if (!zoh) return dt;
  if (a_cont == 0.0) return dt;
  return std::expm1(dt * a_cont) / a_cont;
}

// Scan input u[b, t, d]: x itself, or silu(bias + sum_k w[d,k] x[b, t-K+1+k, d])
// with x taken as zero before the start of the sequence.
double scan_input(const ScanProblem& p, int64_t b, int64_t t, int64_t d) {
  const int64_t L = p.seqlen, D = p.dim;
  if (!p.conv_w) return p.x[(b * L + t) * D + d];
  const int64_t K = p.conv_k;
  double z = p.conv_b ? p.conv_b[d] : 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t src = t - (K - 1) + k;
    if (src < 0) continue;
    z += p.conv_w[d * K + k] * p.x[(b * L + src) * D + d];
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
    const double dt = p.delta[(b * L + t) * D + d];
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
    p.y[(b * L + t) * D + d] = acc + dskip * u;
  }
  if (p.h_last)
    for (int64_t n = 0; n < N; ++n) p.h_last[(b * D + d) * N + n] = h[n];
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

}  // namespace

extern "C" {

// O1: y (batch, L, D) and optionally h_last (batch, D, N) from x, delta
// (batch, L, D), A (D, N), B, C (batch, L, N), Dskip (D) or NULL, h0
// (batch, D, N) or NULL, conv_w (D, K) / conv_b (D) or NULL.  All arrays are
// row-major doubles.  Returns 0, or -1 on a bad argument.  Uses `nthreads`
// std::threads over the (b, d) channels (0 = all hardware threads).
int ssm_ref_scan_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                     const double* x, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* h0, const double* conv_w, const double* conv_b,
                     int64_t conv_k, int zoh, double* y, double* h_last, int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return -1;
  if (conv_w && conv_k < 1) return -1;
  if (batch * dim == 0) return 0;
  if (seqlen > 0 && (!x || !delta || !Bm || !Cm || !y)) return -1;
  if (!A) return -1;
  ScanProblem p{batch, seqlen, dim, dstate, x, delta, A, Bm, Cm, Dskip, h0,
                conv_w, conv_b, conv_k, zoh, y, h_last};
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
// state; y (batch, D) = C . h_new + Dskip * x.  x, delta are (batch, D); B, C
// are (batch, N).  Same recurrence as O1 with L = 1 and no conv prologue.
int ssm_ref_step_f64(int64_t batch, int64_t dim, int64_t dstate, double* h,
                     const double* x, const double* delta, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     int zoh, double* y, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1) return -1;
  if (batch * dim == 0) return 0;
  if (!h || !x || !delta || !A || !Bm || !Cm || !y) return -1;
  // h is both the initial and the final state; the scan reads h0[n] for a
  // channel before it writes h_last[n] of that channel, so in-place is safe.
  return ssm_ref_scan_f64(batch, 1, dim, dstate, x, delta, A, Bm, Cm, Dskip, h,
                          nullptr, nullptr, 0, zoh, y, h, nthreads);
}

}  // extern "C"
