// ssm_bwd.hpp -- gfx950 device code of the backward selective scan.
//
// Gradients of  loss = sum(dy * y) + sum(dh_last * h_last)  for the scan
// without fused steps.  With g_t[n] = d loss / d h_t[n] the chain rule through
//   h_t = a_t h_{t-1} + f_t B_t u_t,   y_t = sum_n C_t h_t + D u_t,
// a_t = exp(Delta_t A), f_t = Delta_t (Delta*B) or (a_t - 1) / A (ZOH) gives
//   g_t        = C_t dy_t + a_{t+1} g_{t+1},          g_{L-1} += dh_last
//   dC_t[n]    = sum_d dy_t h_t[n]                     (sum over channels)
//   dB_t[n]    = sum_d g_t[n] f_t u_t
//   du_t       = sum_n g_t[n] f_t B_t[n] + D dy_t
//   dDelta_t   = sum_n g_t[n] (A a_t h_{t-1} + df/dDelta B_t u_t)
//   dA[n]      = sum_{b,t} g_t[n] (Delta_t a_t h_{t-1} + df/dA B_t u_t)
//   dD         = sum_{b,t} dy_t u_t,      dh0 = a_0 g_0
// The adjoint g obeys the same linear recurrence as h, run backwards in time,
// so it is chunked with the same operator (a, b) o (a', b') (53ai.com
// explainer, section 3.3): a reverse summary per super-chunk, a reverse
// carry walk, and a main pass that starts each super-chunk from its carry.
//
// The main pass needs h_{t-1} at every step, in reverse order.  It takes the
// forward state at every 16th step (kept by the forward scan, or from the
// forward summary and carry passes run at a 16-step chunk), recomputes each
// 16-step chunk forwards into registers and then walks it backwards, so the
// (batch, L, D, N) states are never written to memory (the memory argument
// of the pages' hardware-aware scan: explainer section 3.4).
//
// Layout of the main pass: lane = channel, wave = 4 states (NS) of 64
// channels, workgroup = the N / NS waves of one (batch row, 64-channel tile,
// super-chunk).  Two reductions go through LDS: every 2 steps, over the 64
// channels of a wave (dB, dC; wave-private rows, written as per-tile
// partials), and every 4 steps over the waves of the workgroup (du, dDelta;
// one barrier per 4 steps).  Partials are summed in a fixed order by small
// reduction kernels, so results are deterministic.
#pragma once

#include "ssm_kernels.hpp"

namespace ssmk {

constexpr int kBwdFine = 16;     // recompute chunk (steps held in registers)
constexpr int kBwdBlock = 4;     // steps per LDS exchange
constexpr int kBwdHalf = 8;      // steps whose states are held in registers at once
constexpr int kRedPitch = kWave + 4;   // padded LDS row of the channel sums
static_assert(kBwdFine == kSaveStride, "the forward keeps the states the backward starts from");

struct BwdParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* h0;
  const void* dy;
  const float* dh_last;
  float* dx;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dh0;
  const float* hcar;     // (Bt, Cf-1, D, N) forward state entering fine chunks 1..Cf-1
  float* gsum;           // (Bt, Cs-1, D, N) reverse summaries, then adjoint carries
  float* dsum_s;         // (Bt, Cs-1, D) sums of Delta of super-chunks 1..Cs-1
  float* dAp;            // (Bt * Cs, D, N) per-wave dA partials
  float* dDp;            // (Bt * Cs, D)
  float* dBp;            // (Bt, L, dtiles, N) per-tile dB partials
  float* dCp;            // (Bt, L, dtiles, N)
  float* rgS;            // (Bt, rG, D) grouped reverse walk: sums of Delta per group
  float* rgB;            // (Bt, rG, D, N) adjoint of a group from zero, then its carry in
  int64_t rG, rgsz;      // groups of rgsz super-chunks (rG = 0: one sequential walk)
  int64_t Bt, L, D;
  int64_t Ts;            // super-chunk length (a multiple of kBwdFine)
  int64_t Cs, Cf;        // super-chunks, fine chunks
  int32_t dtiles;
  int32_t nwg;
  float exact_thr;
};

template <int N>
struct BwdLayout {
  static constexpr int NS = N < 4 ? N : 4;   // states per wave
  static constexpr int NG = N / NS;          // waves per workgroup
};

// NS consecutive fp32 values of an LDS row (16-byte aligned for NS = 4).
template <int NS>
__device__ __forceinline__ void lds_row(float (&v)[NS], const float* src) {
  if constexpr (NS == 4) {
    const float4 q = *reinterpret_cast<const float4*>(src);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else if constexpr (NS == 2) {
    const float2 q = *reinterpret_cast<const float2*>(src);
    v[0] = q.x; v[1] = q.y;
  } else {
    v[0] = src[0];
  }
}

// Wave-uniform slow-decay test, as in the forward pass.
template <int NS, int DISC>
__device__ __forceinline__ bool any_exact(const ChanConst<NS, DISC>& cc, float dv) {
  return __builtin_amdgcn_ballot_w64(dv < cc.thr) != 0;
}

// One backward step of one lane for its NS states: given dy, u, Delta and the
// states before (hp) and after (hn) the step, form the gradient terms of the
// step (pB, pC per state; du and dDelta summed over the lane's states, both
// overwritten), add the step's dA terms and move the adjoint g to the
// previous step.  `exact` (wave-uniform) adds to a G, for slow decay, the
// part r G that rounding took from a (r = exp(Delta A) - a, see
// exp_residual); only that product differs between the two forms, so the
// rest of the step is shared code.  SERIES (some state of the wave has |z|
// below series_z) evaluates ZOH's factor f = expm1(z) / A and df/dA, for the
// states with |z| = |Delta A| below series_z, by their series:
//   f = Delta (1 + z/2 + z^2/6 + z^3/24 + z^4/120),
//   df/dA = Delta^2 (1/2 + z/3 + z^2/8 + z^3/30 + z^4/144),
// which also give the A = 0 limits.  The direct forms (a - 1) / A and
// (Delta a - f) / A carry the rounding of a (about 2^-24) divided by the
// difference they take: relative errors of about 2^-24 / |z| in f and
// 2^-23 / z^2 in df/dA (up to twice that with the exp's own rounding; an
// fp32 emulation over random A and Delta at |z| just above the threshold
// found at most 5.8e-5 at 1/16 and 7.8e-4 at 1/64).  The threshold is set
// per input precision so that this stays far inside the tolerance (see
// series_z): 1/16 for fp32 inputs, 1/64 for bf16 (SHORT), where the series
// are cut after their z^2 terms (truncation under 2.5e-7 relative below
// |z| = 1/64; the five-term series hold for |z| < 1/16).
template <bool SHORT>
constexpr float series_z() { return SHORT ? 1.0f / 64.0f : 1.0f / 16.0f; }

template <int NS, int DISC, bool SERIES, bool SHORT>
__device__ __forceinline__ void bwd_lane_step(float (&g)[NS], float (&dA)[NS],
                                              const ChanConst<NS, DISC>& cc,
                                              const float (&Bv)[NS], const float (&Cv)[NS],
                                              const float (&hp)[NS], const float (&hn)[NS],
                                              float u, float dv, float dyv, bool exact,
                                              float (&pB)[NS], float (&pC)[NS], float& du,
                                              float& ddt) {
  float z2[NS], a[NS], G[NS], ag[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    z2[n] = dv * cc.A2[n];
    a[n] = exp2_fast(z2[n]);
    G[n] = fmaf(Cv[n], dyv, g[n]);
  }
  if (exact) {
    // a G plus what rounding took from a (see decay_add)
#pragma unroll
    for (int n = 0; n < NS; ++n) ag[n] = fmaf(a[n], G[n], exp_residual<true>(z2[n], a[n]) * G[n]);
  } else {
#pragma unroll
    for (int n = 0; n < NS; ++n) ag[n] = a[n] * G[n];
  }
  if constexpr (DISC == kDeltaB) {
    // du and dDelta's input term are Delta and u times sum_n G B
    // (A is held as A log2(e); the ln 2 that restores A is applied to the
    // state sum once)
    const float dvu = dv * u;
    float gb = G[0] * Bv[0];
    float dt2 = cc.A2[0] * (ag[0] * hp[0]);
    dA[0] = fmaf(dv, ag[0] * hp[0], dA[0]);
#pragma unroll
    for (int n = 1; n < NS; ++n) {
      const float agh = ag[n] * hp[n];            // shared by dDelta and dA
      gb = fmaf(G[n], Bv[n], gb);
      dt2 = fmaf(cc.A2[n], agh, dt2);
      dA[n] = fmaf(dv, agh, dA[n]);
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) pB[n] = G[n] * dvu;
    du = dv * gb;
    ddt = fmaf(dt2, kLn2, u * gb);
  } else {
    float su = 0.0f, dt2 = 0.0f, dtb = 0.0f;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      float f = (a[n] - 1.0f) * cc.invA[n];
      float dfda = fmaf(dv, a[n], -f) * cc.invA[n];
      if constexpr (SERIES) {
        // some state of the wave has |z| < 1/16: the series there, the direct
        // forms elsewhere (the series is truncated for small |z| only)
        const float z = z2[n] * kLn2;
        float q1, q2;
        if constexpr (SHORT) {
          q1 = fmaf(z, fmaf(z, 1.0f / 6.0f, 0.5f), 1.0f);
          q2 = fmaf(z, fmaf(z, 0.125f, 1.0f / 3.0f), 0.5f);
        } else {
          q1 = fmaf(z, 1.0f / 120.0f, 1.0f / 24.0f);
          q1 = fmaf(z, q1, 1.0f / 6.0f);
          q1 = fmaf(z, q1, 0.5f);
          q1 = fmaf(z, q1, 1.0f);
          q2 = fmaf(z, 1.0f / 144.0f, 1.0f / 30.0f);
          q2 = fmaf(z, q2, 0.125f);
          q2 = fmaf(z, q2, 1.0f / 3.0f);
          q2 = fmaf(z, q2, 0.5f);
        }
        const bool small = fabsf(z) < series_z<SHORT>() || cc.invA[n] == 0.0f;
        f = small ? dv * q1 : f;
        dfda = small ? (dv * dv) * q2 : dfda;
      }
      const float agh = ag[n] * hp[n];
      const float Bu = Bv[n] * u;
      const float Gf = G[n] * f;
      pB[n] = Gf * u;
      su = fmaf(Gf, Bv[n], su);
      dt2 = fmaf(cc.A2[n], agh, dt2);
      dtb = fmaf(ag[n], Bu, dtb);                        // df/dDelta = a
      dA[n] = fmaf(dv, agh, fmaf(G[n] * dfda, Bu, dA[n]));
    }
    du = su;
    ddt = fmaf(dt2, kLn2, dtb);
  }
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    pC[n] = dyv * hn[n];
    g[n] = ag[n];
  }
}

// ---------------------------------------------------------------------------
// reverse summary: per super-chunk s >= 1, the adjoint reaching its first
// step from a zero adjoint past its end, and its sum of Delta
// ---------------------------------------------------------------------------
//
// Latency is hidden as in the forward passes: Delta and dy of the next block
// of kU steps are requested before the current block is folded, and the C
// row of step t - 1 is requested right after the wait for step t's row.
template <int N, typename InT, int DISC>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(4)))
k_bwd_summary(const BwdParams p) {
  constexpr int kU = 8;
  const int wg = xcd_remap(blockIdx.x, p.nwg);
  const int64_t dtile = wg % p.dtiles;
  const int64_t r = wg / p.dtiles;
  const int64_t s = 1 + r % (p.Cs - 1);
  const int64_t b = r / (p.Cs - 1);
  const int64_t dbase = dtile * kWave;
  const uint32_t lo = lane_offset(dbase, p.D);
  const int64_t d = dbase + lo;
  ChanConst<N, DISC> cc;
  load_chan<N, DISC>(cc, p.A + d * N, p.exact_thr);
  const int64_t ts = s * p.Ts;
  const int64_t te = (ts + p.Ts < p.L) ? ts + p.Ts : p.L;
  const int32_t steps = static_cast<int32_t>(te - ts);
  // rows ts .. te-1 of Delta and dy through buffer resources, walked from the
  // last row down
  const int64_t base = (b * p.L + ts) * p.D + dbase;
  const uint32_t row = static_cast<uint32_t>(p.D * sizeof(InT));
  const uint32_t span = static_cast<uint32_t>(steps) * row;
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(static_cast<const InT*>(p.delta) + base, span);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<const InT*>(p.dy) + base, span);
  const uint32_t lo_in = lo * sizeof(InT);
  constexpr InT* kIn = nullptr;
  const InT* Crow = static_cast<const InT*>(p.Cm) + (b * p.L + te - 1) * N;

  float g[N];
#pragma unroll
  for (int n = 0; n < N; ++n) g[n] = 0.0f;
  float dacc = 0.0f, dcomp = 0.0f;   // Kahan sum of Delta
  float Cb0[N], Cb1[N];
  load_row<N>(Cb0, Crow);

  // one step at row offset `off` from the chunk start; the next (earlier)
  // row's C is fetched into Cnext
  auto one_step = [&](float dv, float dyv, bool has_next, float (&Ccur)[N], float (&Cnext)[N]) {
    const InT* nc = Crow - (has_next ? N : 0);
    if constexpr (N >= 2) asm volatile("" : "+s"(nc) : "s"(Ccur[0]));
    load_row<N>(Cnext, nc);
    if (any_exact<N, DISC>(cc, dv)) {   // wave-uniform, as in the forward pass
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float z2 = dv * cc.A2[n];
        const float G = fmaf(Ccur[n], dyv, g[n]);
        const float a = exp2_fast(z2);
        g[n] = fmaf(a, G, exp_residual<true>(z2, a) * G);
      }
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float G = fmaf(Ccur[n], dyv, g[n]);
        g[n] = exp2_fast(dv * cc.A2[n]) * G;
      }
    }
    Crow -= N;
    const float yv = dv - dcomp;
    const float tv = dacc + yv;
    dcomp = (tv - dacc) - yv;
    dacc = tv;
  };

  const int32_t nblk = steps / kU;
  // block k covers steps steps-1-k*kU down to steps-kU-k*kU (offsets from ts)
  auto off_of = [&](int32_t step) { return static_cast<uint32_t>(step) * row; };
  float dc[kU], yc[kU];
  if (nblk > 0) {
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      dc[j] = ldb(rd, lo_in, off_of(steps - 1 - j), kIn);
      yc[j] = ldb(ry, lo_in, off_of(steps - 1 - j), kIn);
    }
  }
  for (int32_t blk = 0; blk < nblk; ++blk) {
    float dn[kU], yn[kU];
    const int32_t nfirst = (blk + 1 < nblk) ? steps - 1 - (blk + 1) * kU : steps - 1 - blk * kU;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      dn[j] = ldb(rd, lo_in, off_of(nfirst - j), kIn);
      yn[j] = ldb(ry, lo_in, off_of(nfirst - j), kIn);
    }
    const int32_t done = blk * kU;
#pragma unroll
    for (int j = 0; j < kU; j += 2) {
      one_step(dc[j], yc[j], done + j + 1 < steps, Cb0, Cb1);
      one_step(dc[j + 1], yc[j + 1], done + j + 2 < steps, Cb1, Cb0);
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) { dc[j] = dn[j]; yc[j] = yn[j]; }
  }
  for (int32_t k = nblk * kU; k < steps; ++k) {
    const int32_t step = steps - 1 - k;
    const float dv = ldb(rd, lo_in, off_of(step), kIn);
    const float dyv = ldb(ry, lo_in, off_of(step), kIn);
    one_step(dv, dyv, k + 1 < steps, Cb0, Cb1);
#pragma unroll
    for (int n = 0; n < N; ++n) Cb0[n] = Cb1[n];
  }
  const int64_t slot = b * (p.Cs - 1) + (s - 1);
  float* gs = p.gsum + (slot * p.D + d) * N;
#pragma unroll
  for (int n = 0; n < N; ++n) gs[n] = g[n];
  p.dsum_s[slot * p.D + d] = dacc - dcomp;
}

// Adjoint carries: one lane per (b, d, n) walks the super-chunks from the
// last to the first; gsum[s - 1] becomes the adjoint entering the end of
// super-chunk s - 1.
template <int N>
__global__ void __launch_bounds__(kWave) k_bwd_combine(const BwdParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * DN) return;
  const int64_t b = idx / DN;
  const int64_t dn = idx - b * DN;
  const int64_t d = dn / N;
  const float a2 = p.A[dn] * kLog2e;
  float carry = p.dh_last ? p.dh_last[idx] : 0.0f;
  const int64_t nc = p.Cs - 1;
  for (int64_t s = nc; s >= 1; --s) {
    const int64_t slot = b * nc + (s - 1);
    const float z2 = a2 * p.dsum_s[slot * p.D + d];
    carry = decay_add(z2, carry, p.gsum[slot * DN + dn]);
    p.gsum[slot * DN + dn] = carry;
  }
}

// The same walk in groups, for few chains over many super-chunks: the
// super-chunks are taken from the last to the first (reversed index r is slot
// Cs - 2 - r), so the forward's walk helpers apply with negative strides.
// Group g of rgsz consecutive reversed super-chunks is folded from zero
// (k_bwd_rgroups), the groups are walked from dh_last (k_bwd_rtop), and each
// group is walked again from its carry, writing the carries (k_bwd_rapply).
template <int N>
__device__ __forceinline__ void rev_walk_ptrs(const BwdParams& p, int64_t b, int64_t d, int64_t dn,
                                              const float** ds, float** hs) {
  const int64_t nc = p.Cs - 1;
  *ds = p.dsum_s + (b * nc + nc - 1) * p.D + d;
  *hs = p.gsum + (b * nc + nc - 1) * p.D * N + dn;
}

template <int N>
__global__ void __launch_bounds__(kWave) k_bwd_rgroups(const BwdParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * p.rG * DN) return;
  const int64_t bg = idx / DN, dn = idx - bg * DN;
  const int64_t b = bg / p.rG, g = bg - b * p.rG;
  const int64_t d = dn / N;
  const int64_t nc = p.Cs - 1;
  const int64_t c0 = g * p.rgsz, c1 = (c0 + p.rgsz < nc) ? c0 + p.rgsz : nc;
  const float* ds;
  float* hs;
  rev_walk_ptrs<N>(p, b, d, dn, &ds, &hs);
  float ssum = 0.0f;
  p.rgB[idx] = walk_chunks<false, true>(p.A[dn] * kLog2e, 0.0f, ds, -p.D, hs, -DN, c0, c1, &ssum);
  if (dn % N == 0) p.rgS[bg * p.D + d] = ssum;
}

template <int N>
__global__ void __launch_bounds__(kWave) k_bwd_rtop(const BwdParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * DN) return;
  const int64_t b = idx / DN, dn = idx - b * DN;
  const int64_t d = dn / N;
  const float carry = p.dh_last ? p.dh_last[idx] : 0.0f;
  walk_carry_in(p.A[dn] * kLog2e, carry, p.rgS + b * p.rG * p.D + d, p.D,
                p.rgB + b * p.rG * DN + dn, DN, p.rG);
}

template <int N>
__global__ void __launch_bounds__(kWave) k_bwd_rapply(const BwdParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * p.rG * DN) return;
  const int64_t bg = idx / DN, dn = idx - bg * DN;
  const int64_t b = bg / p.rG, g = bg - b * p.rG;
  const int64_t d = dn / N;
  const int64_t nc = p.Cs - 1;
  const int64_t c0 = g * p.rgsz, c1 = (c0 + p.rgsz < nc) ? c0 + p.rgsz : nc;
  const float* ds;
  float* hs;
  rev_walk_ptrs<N>(p, b, d, dn, &ds, &hs);
  walk_chunks<true, false>(p.A[dn] * kLog2e, p.rgB[idx], ds, -p.D, hs, -DN, c0, c1, nullptr);
}

// ---------------------------------------------------------------------------
// main backward pass
// ---------------------------------------------------------------------------
template <int N, typename InT, int DISC>
__global__ void __launch_bounds__(kWave * BwdLayout<N>::NG) __attribute__((amdgpu_waves_per_eu(4)))
k_bwd_main(const BwdParams p) {
  constexpr int NS = BwdLayout<N>::NS, NG = BwdLayout<N>::NG;
  constexpr int F = kBwdFine, K = kBwdBlock, H = kBwdHalf;
  static_assert(F % H == 0 && H % K == 0, "halves hold whole blocks");
  // LDS.  Per wave, the dB / dC products of two steps as RR rows of 64
  // channels, [step of the pair][kind][state]; each row is padded to
  // kRedPitch floats, so the LPR lanes summing a row, reading 16 bytes each,
  // touch 16 different bank groups.  The rows are private to the wave, so
  // no workgroup barrier guards them.  Per workgroup, the du / dDelta
  // partials of a block, [buffer][kind][wave][step][lane], double-buffered:
  // one barrier per block separates their writes from their reads.
  constexpr int RR = 4 * NS;           // rows summed together
  constexpr int LPR = kWave / RR;      // lanes per row; each sums RR floats
  static_assert(RR % 4 == 0 && LPR * RR == kWave && K % 2 == 0, "reduction layout");
  __shared__ __attribute__((aligned(16))) float red[NG][RR][kRedPitch];
  __shared__ float xch[2][2][NG][K][kWave];
  // B and C rows.  fp32 rows are read by each wave with scalar loads into
  // SGPRs.  bf16 rows are staged per workgroup: a 16-step chunk's rows,
  // widened to fp32 once, in LDS as [buffer][kind][step][state],
  // double-buffered by chunk (one barrier per chunk separates a fill from
  // its reads); every wave reads its NS states of a row as one broadcast LDS
  // access, and the rows take no SGPRs.  (Measured: staging gains 4% on bf16
  // inputs and loses 3% on fp32, where the scalar rows need no widening.)
  constexpr bool kRowsLds = !std::is_same<InT, float>::value;
  __shared__ __attribute__((aligned(16))) float rows[kRowsLds ? 2 : 1][2][kRowsLds ? F : 1][N];

  const int wg = xcd_remap(blockIdx.x, p.nwg);
  const int64_t dtile = wg % p.dtiles;
  const int64_t r = wg / p.dtiles;
  const int64_t s = r % p.Cs;
  const int64_t b = r / p.Cs;
  // the wave index is uniform across the wave: say so, so that everything
  // derived from it (the B / C row addresses) stays in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int lane = threadIdx.x % kWave;
  const int64_t dbase = dtile * kWave;
  const int64_t d = dbase + lane_offset(dbase, p.D, static_cast<uint32_t>(lane));
  const bool valid = dbase + lane < p.D;   // lanes past D duplicate D - 1 and add nothing
  if (!valid) {
#pragma unroll
    for (int rr = 0; rr < RR; ++rr) red[w][rr][lane] = 0.0f;
  }
  int xb = 0;   // buffer of xch used by the current block (wave-uniform)
  const int n0 = w * NS;

  ChanConst<NS, DISC> cc;
  load_chan<NS, DISC>(cc, p.A + d * N + n0, p.exact_thr);
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  // ZOH's factor is taken from its series when some |Delta A[n]| of the wave
  // is below series_z (see bwd_lane_step)
  constexpr bool kShortSeries = !std::is_same<InT, float>::value;
  float zoh_thr = 0.0f;
  if constexpr (DISC == kZoh) {
    float amin = __builtin_inff();
#pragma unroll
    for (int n = 0; n < NS; ++n) amin = fminf(amin, fabsf(cc.A2[n] * kLn2));
    zoh_thr = amin > 0.0f ? series_z<kShortSeries>() / amin : __builtin_inff();
  }

  // adjoint entering the end of this super-chunk
  float g[NS];
  {
    const float* src = (s == p.Cs - 1)
                           ? (p.dh_last ? p.dh_last + (b * p.D + d) * N + n0 : nullptr)
                           : p.gsum + ((b * (p.Cs - 1) + s) * p.D + d) * N + n0;
#pragma unroll
    for (int n = 0; n < NS; ++n) g[n] = src ? src[n] : 0.0f;
  }
  float dAacc[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) dAacc[n] = 0.0f;
  float dDacc = 0.0f;

  const InT* Bp = static_cast<const InT*>(p.Bm);
  const InT* Cp = static_cast<const InT*>(p.Cm);
  const uint32_t lo = static_cast<uint32_t>(d - dbase);
  const uint32_t lo_in = lo * sizeof(InT), lo_f = lo * 4u;
  const uint32_t row_in = static_cast<uint32_t>(p.D * sizeof(InT));
  const uint32_t row_f = static_cast<uint32_t>(p.D * 4);
  constexpr InT* kIn = nullptr;
  constexpr float* kF = nullptr;

  const int64_t c_lo = s * (p.Ts / F);
  int64_t c_hi = (s + 1) * (p.Ts / F) - 1;
  if (c_hi > p.Cf - 1) c_hi = p.Cf - 1;

  // the chunk rows each thread moves into LDS, loaded one chunk ahead (rows
  // past the sequence are zero; their loads read the last row instead)
  constexpr int kRowVals = kRowsLds ? 2 * F * N : 1;
  constexpr int RV = (kRowVals + kWave * NG - 1) / (kWave * NG);
  float rpre[RV];
  auto rows_load = [&](int64_t cc_) {
    const int64_t tt0 = cc_ * F;
    const int clen = static_cast<int>((tt0 + F < p.L) ? F : p.L - tt0);
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int e = static_cast<int>(threadIdx.x) + i * kWave * NG;
      const int kind = (e / (F * N)) & 1, j = (e / N) % F, n = e % N;
      const InT* src = kind == 0 ? Bp : Cp;
      const float v = ld(src + (b * p.L + tt0 + (j < clen ? j : clen - 1)) * N + n);
      rpre[i] = (e < kRowVals && j < clen) ? v : 0.0f;
    }
  };
  if constexpr (kRowsLds) rows_load(c_hi);
  int rb = 0;   // LDS row buffer of the current chunk (wave-uniform)

  for (int64_t c = c_hi; c >= c_lo; --c) {
    const int64_t t0 = c * F;
    const int len = static_cast<int>((t0 + F < p.L) ? F : p.L - t0);
    // bf16: this chunk's B / C rows into LDS, then the next chunk's requested
    if constexpr (kRowsLds) {
#pragma unroll
      for (int i = 0; i < RV; ++i) {
        const int e = static_cast<int>(threadIdx.x) + i * kWave * NG;
        if (e < kRowVals) (&rows[rb][0][0][0])[e] = rpre[i];
      }
      __syncthreads();
      if (c > c_lo) rows_load(c - 1);
    }
    const float* Brow = &rows[kRowsLds ? rb : 0][0][0][n0];   // + j * N: step j's states
    const float* Crow = &rows[kRowsLds ? rb : 0][1][0][n0];
    // fp32: rows through the scalar cache
    const InT* Bc = static_cast<const InT*>(p.Bm) + (b * p.L + t0) * N + n0;
    const InT* Cc = static_cast<const InT*>(p.Cm) + (b * p.L + t0) * N + n0;
    // this chunk's rows of x, Delta, dy (and dx, dDelta) through buffer
    // resources: constant lane offset, row offsets in SGPRs
    const int64_t base = (b * p.L + t0) * p.D + dbase;
    const uint32_t span_in = static_cast<uint32_t>(len) * row_in;
    const uint32_t span_f = static_cast<uint32_t>(len) * row_f;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const InT*>(p.x) + base, span_in);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(static_cast<const InT*>(p.delta) + base, span_in);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<const InT*>(p.dy) + base, span_in);
    const __amdgpu_buffer_rsrc_t rdx = make_rsrc(p.dx + base, span_f);
    const __amdgpu_buffer_rsrc_t rdd = make_rsrc(p.ddelta + base, span_f);
    // forward state entering the chunk: held in registers for both halves
    // (fp32), or read again at each half's start (bf16, whose LDS rows take
    // the registers)
    const float* h0src = (c == 0) ? (p.h0 ? p.h0 + (b * p.D + d) * N + n0 : nullptr)
                                  : p.hcar + ((b * (p.Cf - 1) + c - 1) * p.D + d) * N + n0;
    float h0c[NS];
    if constexpr (!kRowsLds) {
#pragma unroll
      for (int n = 0; n < NS; ++n) h0c[n] = h0src ? h0src[n] : 0.0f;
    }
    // The chunk is walked back as two halves of H steps, the later half
    // first.  Each half is recomputed forwards from the chunk's entry state
    // (the later half after running through the earlier one), keeping the
    // state before each of its steps: H steps of NS states in registers.
#pragma unroll
    for (int half = F / H - 1; half >= 0; --half) {
      const int j0 = half * H;
      if (j0 >= len) continue;   // wave-uniform
      float h[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) h[n] = kRowsLds ? (h0src ? h0src[n] : 0.0f) : h0c[n];
      float stash[H][NS];
      // x / Delta of K steps at a time, the next K requested before the
      // current K are used.  Row offsets are clamped to the chunk's last row
      // (the rows past it are never used; this keeps every access in bounds
      // whether or not the descriptor's range check covers the SGPR offset).
      auto roff = [&](int j) { return static_cast<uint32_t>(j < len ? j : len - 1) * row_in; };
      float xa[K], da[K];
#pragma unroll
      for (int jj = 0; jj < K; ++jj) {
        xa[jj] = ldb(rx, lo_in, roff(jj), kIn);
        da[jj] = ldb(rd, lo_in, roff(jj), kIn);
      }
#pragma unroll
      for (int jb = 0; jb < (j0 + H) / K; ++jb) {
        float xn[K], dn[K];
        const int nb = (jb + 1 < (j0 + H) / K) ? jb + 1 : jb;
#pragma unroll
        for (int jj = 0; jj < K; ++jj) {
          xn[jj] = ldb(rx, lo_in, roff(nb * K + jj), kIn);
          dn[jj] = ldb(rd, lo_in, roff(nb * K + jj), kIn);
        }
        float Bb[K][NS];
        if constexpr (!kRowsLds) {
#pragma unroll
          for (int jj = 0; jj < K; ++jj) {
            const int j = jb * K + jj;
            load_row<NS>(Bb[jj], Bc + (j < len ? j : len - 1) * N);
          }
        }
#pragma unroll
        for (int jj = 0; jj < K; ++jj) {
          const int j = jb * K + jj;
          float Bv[NS];
          if constexpr (kRowsLds) {
            lds_row<NS>(Bv, Brow + j * N);
          } else {
#pragma unroll
            for (int n = 0; n < NS; ++n) Bv[n] = Bb[jj][n];
          }
          if (j >= j0) {
#pragma unroll
            for (int n = 0; n < NS; ++n) stash[j - j0][n] = h[n];
          }
          if (j < len) {
            if (any_exact<NS, DISC>(cc, da[jj]))
              ssm_step_lane<NS, DISC, false, true, true>(h, cc, Bv, Bv, xa[jj], da[jj]);
            else
              ssm_step_lane<NS, DISC, false, false>(h, cc, Bv, Bv, xa[jj], da[jj]);
          }
        }
#pragma unroll
        for (int jj = 0; jj < K; ++jj) {
          xa[jj] = xn[jj];
          da[jj] = dn[jj];
        }
      }
      // h is now the state after the half's last step

    // walk the half back in blocks of K steps
#pragma unroll
    for (int jb = (j0 + H) / K - 1; jb >= j0 / K; --jb) {
      if (jb * K >= len) continue;   // wave-uniform
      // the block's x / Delta / dy (and fp32 B / C) rows, all requested
      // before the first is used (bf16 B / C rows are read from LDS at the
      // step)
      float ub[K], db[K], yb[K], Bb[K][NS], Cb[K][NS];
#pragma unroll
      for (int jj = 0; jj < K; ++jj) {
        const int j = jb * K + jj;
        const uint32_t off = static_cast<uint32_t>(j < len ? j : len - 1) * row_in;
        ub[jj] = ldb(rx, lo_in, off, kIn);
        db[jj] = ldb(rd, lo_in, off, kIn);
        yb[jj] = ldb(ry, lo_in, off, kIn);
        if constexpr (!kRowsLds) {
          load_row<NS>(Bb[jj], Bc + (j < len ? j : len - 1) * N);
          load_row<NS>(Cb[jj], Cc + (j < len ? j : len - 1) * N);
        }
      }
      // keep the scalar row loads here, together (one wait for the block)
      // rather than sunk next to each step's first use
      if constexpr (!kRowsLds && NS == 4) {
#pragma unroll
        for (int jj = 0; jj < K; ++jj)
          asm volatile("" ::"s"(Bb[jj][0]), "s"(Bb[jj][1]), "s"(Bb[jj][2]), "s"(Bb[jj][3]),
                       "s"(Cb[jj][0]), "s"(Cb[jj][1]), "s"(Cb[jj][2]), "s"(Cb[jj][3]));
      }
#pragma unroll
      for (int jj = K - 1; jj >= 0; --jj) {
        const int j = jb * K + jj;
        float pB[NS], pC[NS], du = 0.0f, ddt = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) pB[n] = pC[n] = 0.0f;
        const float u = ub[jj], dv = db[jj], dyv = yb[jj];
        float Bv[NS], Cv[NS];
        if constexpr (kRowsLds) {
          lds_row<NS>(Bv, Brow + j * N);
          lds_row<NS>(Cv, Crow + j * N);
        } else {
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            Bv[n] = Bb[jj][n];
            Cv[n] = Cb[jj][n];
          }
        }
        if (j < len) {
          const int js = j - j0;                    // index within the half
          // the state after step js: the stash holds the state before every
          // step of the half, and past a short half's last step the state
          // after it (the recompute stashes before it skips a step)
          float hn[NS];
#pragma unroll
          for (int n = 0; n < NS; ++n) hn[n] = (js + 1 < H) ? stash[js + 1 < H ? js + 1 : js][n] : h[n];
          // wave-uniform forms: slow decay, and (ZOH) small |Delta A| series
          const bool exact = any_exact<NS, DISC>(cc, dv);
          const bool series = DISC == kZoh && __builtin_amdgcn_ballot_w64(dv < zoh_thr) != 0;
          if (series)
            bwd_lane_step<NS, DISC, true, kShortSeries>(g, dAacc, cc, Bv, Cv, stash[js], hn, u,
                                                        dv, dyv, exact, pB, pC, du, ddt);
          else
            bwd_lane_step<NS, DISC, false, kShortSeries>(g, dAacc, cc, Bv, Cv, stash[js], hn, u,
                                                         dv, dyv, exact, pB, pC, du, ddt);
          dDacc = fmaf(dyv, u, dDacc);   // every wave sums it; wave 0 stores it
        }
        const int sp = jj & 1;   // the pair (jj | 1, jj & ~1) shares the rows
        if (valid) {   // lanes past the last channel keep their zero entries
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            red[w][(sp * 2 + 0) * NS + n][lane] = pB[n];
            red[w][(sp * 2 + 1) * NS + n][lane] = pC[n];
          }
        }
        xch[xb][0][w][jj][lane] = du;
        xch[xb][1][w][jj][lane] = ddt;
        if (sp == 0) {
          // dB / dC of steps jj + 1 and jj: LPR lanes sum each row over the
          // wave's 64 channels (the wave's own LDS writes are seen in order)
          __builtin_amdgcn_wave_barrier();
          const int rr = lane / LPR, c = lane % LPR;
          const float4* src = reinterpret_cast<const float4*>(&red[w][rr][c * RR]);
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < RR / 4; ++i) {
            const float4 v = src[i];
            acc += v.x;
            acc += v.y;
            acc += v.z;
            acc += v.w;
          }
          if constexpr (LPR >= 2)   // quad_perm [1, 0, 3, 2]
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xF, 0xF, false));
          if constexpr (LPR >= 4)   // quad_perm [2, 3, 0, 1]
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xF, 0xF, false));
          if constexpr (LPR >= 8)   // row_half_mirror
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x141, 0xF, 0xF, false));
          if constexpr (LPR >= 16)  // row_mirror
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x140, 0xF, 0xF, false));
          const int jr = jj + rr / (2 * NS);
          const int kind = (rr / NS) & 1;
          const int n = rr % NS;
          if (c == 0 && jb * K + jr < len) {
            float* dst = kind == 0 ? p.dBp : p.dCp;
            dst[((b * p.L + t0 + jb * K + jr) * p.dtiles + dtile) * N + n0 + n] = acc;
          }
          __builtin_amdgcn_wave_barrier();   // the reads stay ahead of the next pair's writes
        }
      }
      __syncthreads();
      // du / dDelta: wave w finishes steps jj = w, w + NG, ...
#pragma unroll
      for (int jj = w; jj < K; jj += NG) {
        const int j = jb * K + jj;
        if (j < len) {
          float su = 0.0f, sd = 0.0f;
#pragma unroll
          for (int v = 0; v < NG; ++v) {
            su += xch[xb][0][v][jj][lane];
            sd += xch[xb][1][v][jj][lane];
          }
          const float dyv = ldb(ry, lo_in, j * row_in, kIn);
          stb(rdx, lo_f, j * row_f, fmaf(dsk, dyv, su), kF);
          stb(rdd, lo_f, j * row_f, sd, kF);
        }
      }
      xb ^= 1;   // the next block's exchange goes to the other buffer
    }
    }
    rb ^= 1;     // the next chunk's rows go to the other buffer
  }
  const int64_t slot = b * p.Cs + s;
#pragma unroll
  for (int n = 0; n < NS; ++n) p.dAp[(slot * p.D + d) * N + n0 + n] = dAacc[n];
  if (w == 0) p.dDp[slot * p.D + d] = dDacc;
  if (s == 0 && p.dh0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) p.dh0[(b * p.D + d) * N + n0 + n] = g[n];
  }
}

// dB, dC: sum the per-tile partials (one thread per (b, t, n)).
template <int N>
__global__ void __launch_bounds__(256) k_bwd_reduce_bc(const BwdParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = p.Bt * p.L * N;
  if (i >= total) return;
  const int64_t bt = i / N, n = i - bt * N;
  const float* sb = p.dBp + bt * p.dtiles * N + n;
  const float* sc = p.dCp + bt * p.dtiles * N + n;
  float ab = 0.0f, ac = 0.0f;
  for (int k = 0; k < p.dtiles; ++k) {
    ab += sb[k * N];
    ac += sc[k * N];
  }
  p.dB[i] = ab;
  p.dC[i] = ac;
}

// dA (D, N) and dD (D): sum the per-wave partials over batch rows and
// super-chunks.  A workgroup covers 64 consecutive outputs (of dA, then dD);
// its 16 waves sum every 16th partial each and wave 0 adds the 16 results in
// a fixed order, so the sum is deterministic.
constexpr int kRedWaves = 16;

template <int N>
__global__ void __launch_bounds__(kWave * kRedWaves) k_bwd_reduce_ad(const BwdParams p) {
  __shared__ float part[kRedWaves][kWave];
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kWave + lane;
  const int64_t DN = p.D * N;
  const int64_t parts = p.Bt * p.Cs;
  const bool isA = i < DN;
  const bool isD = !isA && i < DN + p.D && p.dD;
  float acc = 0.0f;
  if (isA) {
    for (int64_t k = w; k < parts; k += kRedWaves) acc += p.dAp[k * DN + i];
  } else if (isD) {
    for (int64_t k = w; k < parts; k += kRedWaves) acc += p.dDp[k * p.D + (i - DN)];
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int v = 0; v < kRedWaves; ++v) sum += part[v][lane];
    if (isA) p.dA[i] = sum;
    else if (isD) p.dD[i - DN] = sum;
  }
}

}  // namespace ssmk
