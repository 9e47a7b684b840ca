// ssm_kernels.hpp -- gfx950 device code of the selective state-space scan.
//
// Work decomposition of the scan (its kernels use one 64-lane wave per
// workgroup; the decode step and the backward pass have their own layouts):
//   * lane  = one channel (b, d); the lane keeps all N states of that channel
//     in VGPRs for the whole chunk, so the expanded (batch, L, D, N) state is
//     never written anywhere (the memory argument of the pages'
//     "hardware-aware" scan: 53ai.com explainer section 3.4; VMamba note,
//     section "硬件感知的设计");
//   * wave  = 64 consecutive channels of one batch row and one time chunk;
//     x, Delta, y are read/written as 64 consecutive elements per time step
//     (one coalesced 128/256-byte row), while B[b,t,:] and C[b,t,:] are the
//     same for every lane of the wave and are fetched with scalar loads into
//     SGPRs, so they cost no vector-memory or VGPR bandwidth;
//   * chunk = a slice of the time axis.  When batch * D alone does not fill the
//     GPU, the time axis is cut into chunks scanned in parallel:
//       k_chunk_summary  per chunk, the state reached from a zero state and
//                        the chunk's total step sum(Delta);
//       k_carry_combine  per (b, d, n), the carries into every chunk by the
//                        associative operator (a, b) o (a', b') = (a a', a' b + b')
//                        (53ai.com explainer section 3.3: split the sequence,
//                        scan the parts, combine and adjust); long chains of
//                        few (b, d, n) are walked in groups instead;
//       k_scan_out       per chunk, the recurrence again from its carry-in,
//                        writing y (and h_last from the final chunk, and
//                        optionally the state every 16 steps for the
//                        backward pass).
//     The chunk's decay factor is exp(A * sum Delta), the product of its
//     per-step Abar factors.
//
// Arithmetic per element (b, t, d, n), Delta*B discretization:
//     a = exp2(Delta * A[n] * log2 e)       v_mul + v_exp (half rate)
//     h = a * h + (Delta * u) * B[n]        v_mul + v_fma
//     y += C[n] * h                         v_fma
// The ZOH discretization uses h' = a (h + q) - q with q = u B[n] / A[n], which
// equals a h + (a - 1) q.
//
// Fused around the scan (all optional): the step size from its
// pre-activation, Delta = softplus(delta + bias[d]), applied as each block of
// Delta values becomes current; the output gate y * silu(z), z streamed like
// x; and the conv window taken from / handed back to a caller's conv state.
//
// Slow decay.  When |Delta A| is tiny, Abar = exp(Delta A) lies so close to 1
// that rounding it to fp32 biases the decay rate by up to 2^-24 / |Delta A|,
// and with a steady Delta that bias compounds over the whole memory horizon.
// At any step where some lane has min_n |Delta A[n]| below a threshold, the
// wave adds back what rounding took from Abar: with r = exp(Delta A) - Abar,
// from the expm1 series where |Delta A| < 1/16 and 0 elsewhere, it steps
// h' = Abar h + (r h + Bbar u).  A strong decay thus stays the direct product
// Abar h (no h + expm1 h that would cancel to a rounding error of the size of
// the old h), with no per-state choice between two forms.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssmk {

using bf16_t = uint16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;
constexpr int kConvTaps = 4;   // the conv prologue always runs 4 taps; shorter
                               // filters are zero-padded at the oldest taps

enum Disc : int { kDeltaB = 0, kZoh = 1 };

struct ScanParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  const float* h0;
  float* h_last;
  void* y;
  const float* conv_w;   // (D, conv_k)
  const float* conv_b;
  float* dsum;           // (Bt, C-1, D)       chunk sums of Delta
  float* hsum;           // (Bt, C-1, D, N)    chunk end states, then carries
  int64_t Bt, L, D;
  int64_t T;             // chunk length
  int64_t C;             // number of chunks
  int32_t dtiles;        // ceil(D / 64)
  int32_t conv_k;
  int32_t nwg;           // workgroups in the launch (for the XCD remap)
  float exact_thr;       // min |Delta A| below this takes the slow-decay form
  const float* dt_bias;  // (D) or null
  int32_t dt_mode;       // kDtRaw, kDtBias or kDtSoftplus
  const void* z;         // (Bt, L, D) gate or null
  const float* cs_in;    // (Bt, D, conv_k - 1) conv window before token 0, or null
  float* cs_out;         // (Bt, D, conv_k - 1) last conv_k - 1 inputs, or null
  // grouped carry walk (long chunk chains): G groups of gsz chunks
  float* gS;             // (Bt, G, D)     group sums of Delta
  float* gB;             // (Bt, G, D, N)  group end states from zero, then carries into groups
  int64_t G, gsz;
  // states kept for the backward pass: the state entering every
  // kSaveStride-th step, (Bt, nsave, D, N), or null
  float* hsave;
  int64_t nsave;
};

// Steps between the states the output pass keeps for the backward pass.
constexpr int kSaveStride = 16;

// How the step size is formed from the given delta values.
enum DtMode : int { kDtRaw = 0, kDtBias = 1, kDtSoftplus = 2 };

struct StepParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dskip;
  float* h;
  void* y;
  int64_t Bt, D;
  int32_t dtiles;
  int32_t nwg;
  float exact_thr;
  const float* dt_bias;
  int32_t dt_mode;
  int32_t conv_k;        // 0 = no conv
  const void* z;         // (Bt, D) gate or null
  const float* conv_w;   // (D, conv_k)
  const float* conv_b;
  float* conv_state;     // (Bt, D, conv_k - 1), updated in place
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(bf16_t* p, float v) {
  // round to nearest even (gfx950 has a native conversion for this)
  *p = __builtin_bit_cast(bf16_t, static_cast<__bf16>(v));
}

// Rows of B and C are identical across the wave: fetch them through the
// constant address space so the compiler emits scalar loads into SGPRs.
typedef const float __attribute__((address_space(4)))* const_f32_ptr;
typedef const uint32_t __attribute__((address_space(4)))* const_u32_ptr;

template <int N>
__device__ __forceinline__ void load_row(float (&r)[N], const float* p) {
  const_f32_ptr q = (const_f32_ptr)(p);
#pragma unroll
  for (int n = 0; n < N; ++n) r[n] = q[n];
}

template <int N>
__device__ __forceinline__ void load_row(float (&r)[N], const bf16_t* p) {
  if constexpr (N == 1) {
    // a single bf16 per row: a 16-bit vector load (a dword scalar load could
    // run 2 bytes past the end of the array)
    r[0] = ld(p);
  } else {
    const_u32_ptr q = (const_u32_ptr)(p);
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      const uint32_t w = q[k];
      r[2 * k] = __uint_as_float(w << 16);
      r[2 * k + 1] = __uint_as_float(w & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ __forceinline__ float silu(float z) {
  // z / (1 + exp(-z)); for z -> -inf the exp overflows to inf and rcp gives 0
  const float e = exp2_fast(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// softplus(v) = log(1 + exp(v)) = max(v, 0) + log1p(e), e = exp(-|v|) in
// (0, 1].  log1p(e) is taken as log(w) * e / (w - 1) with w = 1 + e rounded
// (Goldberg's correction for the rounding of w), and as e itself once w
// rounds to 1, so the result keeps full relative precision far into the
// negative tail, where softplus(v) ~ exp(v).
__device__ __forceinline__ float softplus(float v) {
  const float e = exp2_fast(-fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  const float l =
      (w == 1.0f) ? e : (__builtin_amdgcn_logf(w) * kLn2) * (e * __builtin_amdgcn_rcpf(w - 1.0f));
  return fmaxf(v, 0.0f) + l;
}

// The step size from a given delta value and the channel's bias.
__device__ __forceinline__ float dt_transform(float v, float bias, int mode) {
  v += bias;
  return mode == kDtSoftplus ? softplus(v) : v;
}

// Workgroups are handed to the 8 XCDs round-robin (id i on XCD i % 8).  Map
// them so that each XCD receives one contiguous range of logical ids, which
// keeps the waves sharing a (batch, chunk) -- and its B/C rows -- in one L2.
__device__ __forceinline__ int xcd_remap(int i, int nwg) {
  const int x = i & 7, k = i >> 3;
  const int q = nwg >> 3, r = nwg & 7;
  return x * q + (x < r ? x : r) + k;
}

// Per-lane constants of one channel.
template <int N, int DISC>
struct ChanConst {
  float A2[N];     // A[d,n] * log2(e)
  float invA[N];   // 1 / A[d,n] (0 where A is 0); ZOH only
  float thr;       // Delta below thr means some |Delta A[n]| is below the threshold
};

template <int N, int DISC>
__device__ __forceinline__ void load_chan(ChanConst<N, DISC>& cc, const float* Arow,
                                          float thr_scale) {
  float amin = __builtin_inff();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float a = Arow[n];
    cc.A2[n] = a * kLog2e;
    if constexpr (DISC == kZoh) cc.invA[n] = (a != 0.0f) ? 1.0f / a : 0.0f;
    amin = fminf(amin, fabsf(a));
  }
  // min_n |Delta A[n]| < thr_scale  <=>  Delta < thr_scale / min_n |A[n]|
  cc.thr = (amin > 0.0f) ? thr_scale / amin : __builtin_inff();
}

// exp(z) - a given z2 = z * log2(e) and a = exp2(z2), the part of exp(z)
// that rounding a to fp32 lost.  Below |z| = 1/16 it is (1 - a) + expm1(z),
// with 1 - a exact (a lies within [1/2, 2]) and expm1 from its series
// z (1 + z/2 + z^2/6 + z^3/24 + z^4/120) (truncation error under 4e-11
// relative); above it, 0 (a is then within ~1e-6 of exp(z) relative to 1 - a).
//
// Two evaluations of the same value.  SELECT picks between the series and 0
// with a compare.  The default takes the series at z clamped to
// [-1/16, 1/16] and multiplies it by a factor that is exactly 1 for
// |z| < 1/16 and exactly 0 otherwise: 2^40 (1/16 - |z|) clamped to [0, 1]
// (fp32 values of |z| differ from 1/16 by 2^-28 or more, so the product is
// never strictly between 0 and 1).  It needs no compare, hence no lane-mask
// registers, which the unrolled steps otherwise hold one per state.  Which
// compiles to faster code depends on the kernel around it (measured: the
// clamped form in the forward passes, the select in the backward pass).
template <bool SELECT = false>
__device__ __forceinline__ float exp_residual(float z2, float a) {
  const float z = z2 * kLn2;
  const float zs = SELECT ? z : __builtin_amdgcn_fmed3f(z, -0.0625f, 0.0625f);
  float p = fmaf(zs, 1.0f / 120.0f, 1.0f / 24.0f);
  p = fmaf(zs, p, 1.0f / 6.0f);
  p = fmaf(zs, p, 0.5f);
  p = fmaf(zs, p, 1.0f);
  if constexpr (SELECT) {
    return (fabsf(z) < 0.0625f) ? fmaf(z, p, 1.0f - a) : 0.0f;
  } else {
    const float m = __builtin_amdgcn_fmed3f(fmaf(-fabsf(z), 0x1p40f, 0x1p36f), 0.0f, 1.0f);
    return fmaf(zs, p, 1.0f - a) * m;
  }
}

// The A a scaled ZOH state runs with: A itself, except that |A| below 2^-60
// (A = 0 included) becomes -2^-60 (keeping a positive A's sign).  A h then
// stays in fp32's normal range wherever h does, down to |h| ~ 2^-66, and
// can be divided out again; the substitution changes exp(Delta A) by about
// Delta 2^-60 and (exp(Delta A) - 1) / A, the input factor, by a relative
// Delta 2^-61: far below fp32 resolution for any Delta a model uses.  (Such
// a tiny |Delta A| always takes the slow-decay form, whose series keeps both
// exact.)  The scaled state assumes |A h| stays below fp32's overflow limit.
__device__ __forceinline__ float scaled_a(float A) {
  return (A > 0.0f) ? fmaxf(A, 0x1p-60f) : fminf(A, -0x1p-60f);
}

// One time step for one lane: updates h[] and returns sum_n C[n] h[n].
// u is the scan input, dv = Delta.  WITH_Y = false skips the readout.
// EXACT selects the slow-decay form (see the header); SELECT the evaluation
// of its residual (see exp_residual).
//
// SCALED (ZOH without readout) carries g = A h in place of h.  With Bbar =
// (Abar - 1) / A B the step becomes g' = Abar g + (Abar - 1) B u, evaluated
// as Abar (g + B u) - B u: three operations per state where h takes four
// (two products form (B u) / A).  The caller converts g back to h, and runs
// it with A replaced by scaled_a(A).
template <int N, int DISC, bool WITH_Y, bool EXACT, bool SELECT = false, bool SCALED = false>
__device__ __forceinline__ float ssm_step_lane(float (&h)[N], const ChanConst<N, DISC>& cc,
                                               const float (&Bv)[N], const float (&Cv)[N],
                                               float u, float dv) {
  static_assert(!SCALED || (DISC == kZoh && !WITH_Y), "the scaled state is ZOH's, without readout");
  float acc0 = 0.0f, acc1 = 0.0f;
  const float du = dv * u;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float z2 = dv * cc.A2[n];
    const float a = exp2_fast(z2);
    if constexpr (SCALED) {
      const float bu = u * Bv[n];
      if constexpr (!EXACT) {
        h[n] = fmaf(a, h[n] + bu, -bu);
      } else {
        const float r = exp_residual<SELECT>(z2, a);
        h[n] = fmaf(a, h[n], fmaf((a - 1.0f) + r, bu, r * h[n]));   // (a - 1) + r = expm1
      }
    } else if constexpr (!EXACT) {
      if constexpr (DISC == kDeltaB) {
        h[n] = fmaf(a, h[n], du * Bv[n]);
      } else {
        const float q = (u * Bv[n]) * cc.invA[n];
        h[n] = fmaf(a, h[n] + q, -q);
      }
    } else {
      const float r = exp_residual<SELECT>(z2, a);
      float gu;   // the input factor times u
      if constexpr (DISC == kDeltaB) {
        gu = du;
      } else {
        const float e = (a - 1.0f) + r;   // expm1(Delta A)
        gu = (cc.invA[n] != 0.0f) ? (e * cc.invA[n]) * u : du;   // A = 0: limit Delta
      }
      h[n] = fmaf(a, h[n], fmaf(gu, Bv[n], r * h[n]));
    }
    if constexpr (WITH_Y) {
      if (n & 1) acc1 = fmaf(Cv[n], h[n], acc1);
      else acc0 = fmaf(Cv[n], h[n], acc0);
    }
  }
  return acc0 + acc1;
}

template <int N, int DISC, bool WITH_Y, bool SCALED = false>
__device__ __forceinline__ float ssm_step_any(float (&h)[N], const ChanConst<N, DISC>& cc,
                                              const float (&Bv)[N], const float (&Cv)[N],
                                              float u, float dv) {
  // wave-uniform choice: the fast form unless some lane has a tiny |Delta A|
  if (__builtin_amdgcn_ballot_w64(dv < cc.thr) != 0)
    return ssm_step_lane<N, DISC, WITH_Y, true, false, SCALED>(h, cc, Bv, Cv, u, dv);
  return ssm_step_lane<N, DISC, WITH_Y, false, false, SCALED>(h, cc, Bv, Cv, u, dv);
}

// Causal conv window: taps w[0..3] (oldest .. newest, zero-padded at the
// oldest end for K < 4) and the previous three inputs.
struct ConvState {
  float w0, w1, w2, w3, bias;
  float xm3, xm2, xm1;   // x[t-3], x[t-2], x[t-1]
};

template <typename InT>
__device__ __forceinline__ void conv_init(ConvState& cs, const ScanParams& p, int64_t b,
                                          int64_t d, int64_t t0) {
  const int K = p.conv_k;
  float w[kConvTaps] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; ++k) w[kConvTaps - K + k] = p.conv_w[d * K + k];
  cs.w0 = w[0]; cs.w1 = w[1]; cs.w2 = w[2]; cs.w3 = w[3];
  cs.bias = p.conv_b ? p.conv_b[d] : 0.0f;
  const InT* xp = static_cast<const InT*>(p.x);
  const int64_t base = b * p.L;
  // x[t] for t = t0 - 3 .. t0 - 1; before token 0 from the caller's window
  // (x[-S .. -1] = cs_in[b, d, 0 .. S-1]), or zero
  const int S = K - 1;
  const float* win = p.cs_in ? p.cs_in + (b * p.D + d) * S : nullptr;
  float xm[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int64_t t = t0 - 3 + k;
    if (t >= 0) xm[k] = ld(xp + (base + t) * p.D + d);
    else xm[k] = (win && t >= -S) ? win[S + t] : 0.0f;
  }
  cs.xm3 = xm[0];
  cs.xm2 = xm[1];
  cs.xm1 = xm[2];
}

// The last K - 1 inputs of the window, oldest first, into out[0 .. K-2].
__device__ __forceinline__ void conv_save(const ConvState& cs, int K, float* out) {
  const float xm[3] = {cs.xm3, cs.xm2, cs.xm1};
  const int S = K - 1;
  for (int j = 0; j < S; ++j) out[j] = xm[3 - S + j];
}

__device__ __forceinline__ float conv_push(ConvState& cs, float xv) {
  float z = fmaf(cs.w3, xv, cs.bias);
  z = fmaf(cs.w2, cs.xm1, z);
  z = fmaf(cs.w1, cs.xm2, z);
  z = fmaf(cs.w0, cs.xm3, z);
  cs.xm3 = cs.xm2; cs.xm2 = cs.xm1; cs.xm1 = xv;
  return silu(z);
}

// Lane offset within a 64-channel tile, clamped so that lanes past the last
// channel duplicate channel D - 1.  `l` is the lane within its wave (the
// thread index in the one-wave workgroups of the forward kernels).
__device__ __forceinline__ uint32_t lane_offset(int64_t dbase, int64_t D,
                                                uint32_t l = threadIdx.x) {
  const int64_t last = D - 1 - dbase;
  return (static_cast<int64_t>(l) <= last) ? l : static_cast<uint32_t>(last);
}

// Decompose a (remapped) workgroup id of the chunked grid.
struct Tile {
  int64_t b, chunk, dtile;
};

__device__ __forceinline__ Tile tile_of(int wg, int64_t dtiles, int64_t nchunks) {
  Tile t;
  t.dtile = wg % dtiles;
  const int64_t r = wg / dtiles;
  t.chunk = r % nchunks;
  t.b = r / nchunks;
  return t;
}

// ---------------------------------------------------------------------------
// the time loop shared by the summary and output passes
// ---------------------------------------------------------------------------

// Time steps whose x / Delta loads are batched (and prefetched one batch
// ahead): the summary pass does less arithmetic per step, so it looks
// further ahead to cover the same memory latency.
constexpr int kUnrollOut = 4;
static_assert(kSaveStride % kUnrollOut == 0, "kept states fall on block ends");
constexpr int kUnrollSum = 8;   // (4 and 6 measured the same on the fp32, conv and long scans)

// Streams through buffer resources: the wave-uniform chunk base and size sit
// in an SGPR descriptor, the lane's byte offset is a constant VGPR and the
// row's byte offset an SGPR advanced with scalar adds, so the vector memory
// instructions need no per-lane address arithmetic at all.  Accesses past
// the descriptor's size return 0 / are dropped by the hardware.
constexpr int kBufferFlags = 0x00020000;   // gfx9-family raw buffer, 32-bit data

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const T* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufferFlags);
}

__device__ __forceinline__ float ldb(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                     float*) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ float ldb(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                     bf16_t*) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0))
                         << 16);
}
// Row stores (y in the output pass, dx and dDelta in the backward) are
// non-temporal (cache policy kCpolNt): nothing in the pass reads them again,
// so they need not take cache lines from the inputs (the output pass reads
// x and Delta a second time, after the summary pass).  Measured on the 8 x 2048 x
// 1536 x 16 fp32 scan: 169-174 -> 160-166 us; bf16 shapes and the backward
// unchanged.  Non-temporal loads of the output pass's x and Delta, their last
// reader, lost part of that again, so loads keep the default policy.
constexpr int kCpolNt = 2;
__device__ __forceinline__ void stb(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                    float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, kCpolNt);
}
__device__ __forceinline__ void stb(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                    float v, bf16_t*) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(bf16_t, static_cast<__bf16>(v)), r,
                                        voff, soff, kCpolNt);
}

// Lanes past the last channel (D not a multiple of 64) run channel D - 1
// again: they read the same inputs and produce bit-identical results, so all
// stores can be unconditional (duplicate stores of equal values to one
// address) and no branch splits the wave.
//
// Scalar-load schedule: the B and C rows of step t + 1 are requested at the
// top of step t into the second of two row buffers, so a whole step of
// arithmetic covers their latency.  (Scalar loads complete out of order, so
// the only usable wait is "all outstanding"; it falls at the top of the next
// step, after the loads had a full step to land.)
//
// GATE (output pass only) streams z like x and multiplies each output by
// silu(z).  SAVE (output pass only) writes the state entering every
// kSaveStride-th step to p.hsave.  cs_save, when not null, receives the conv window after the last
// step (the caller passes it for the final chunk only).  SCALED (ZOH summary
// pass, from a zero state) carries A h through the chunk (see ssm_step_lane)
// and converts it back to h after the last step.
template <int N, typename InT, typename OutT, int DISC, bool CONV, bool OUT, bool GATE,
          bool SAVE = false, bool SCALED = false>
__device__ __forceinline__ void chunk_loop(const ScanParams& p, int64_t b, int64_t dbase,
                                           uint32_t lo, int64_t t0, int32_t steps, float (&h)[N],
                                           float* dsum_out, float* cs_save) {
  static_assert(OUT || !GATE, "the gate applies to the output pass");
  static_assert(OUT || !SAVE, "the output pass keeps the states");
  static_assert(!SCALED || (!OUT && DISC == kZoh), "the scaled state is the ZOH summary's");
  // (the conv prologue's extra registers would push an 8-step summary block
  // past 128 VGPRs, so conv summaries prefetch 6 steps ahead)
  constexpr int kU = OUT ? kUnrollOut : (CONV ? 6 : kUnrollSum);
  const int64_t d = dbase + lo;
  ChanConst<N, DISC> cc;
  load_chan<N, DISC>(cc, p.A + d * N, p.exact_thr);
  if constexpr (SCALED) {
#pragma unroll
    for (int n = 0; n < N; ++n) cc.A2[n] = scaled_a(p.A[d * N + n]) * kLog2e;
  }
  const float dsk = (OUT && p.Dskip) ? p.Dskip[d] : 0.0f;
  const int dtm = p.dt_mode;
  const float dtb = (dtm != kDtRaw && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  ConvState cs;
  if constexpr (CONV) conv_init<InT>(cs, p, b, d, t0);

  const int64_t D = p.D;
  const uint32_t lo_in = lo * sizeof(InT);
  const uint32_t lo_out = lo * sizeof(OutT);
  // x, Delta (and y) of this wave's chunk: rows of D elements starting at
  // (b, t0, dbase); the plan keeps steps * D * 4 bytes below 2^31
  const int64_t chunk_base = (b * p.L + t0) * D + dbase;
  const uint32_t row_in = static_cast<uint32_t>(D * sizeof(InT));
  const uint32_t span_in = static_cast<uint32_t>(steps) * row_in;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const InT*>(p.x) + chunk_base, span_in);
  const __amdgpu_buffer_rsrc_t rd =
      make_rsrc(static_cast<const InT*>(p.delta) + chunk_base, span_in);
  const __amdgpu_buffer_rsrc_t rz =
      make_rsrc(static_cast<const InT*>(GATE ? p.z : p.x) + chunk_base, GATE ? span_in : 0u);
  const uint32_t row_out = static_cast<uint32_t>(D * sizeof(OutT));
  // (the summary pass writes no y: its descriptor then covers nothing)
  const __amdgpu_buffer_rsrc_t ry =
      make_rsrc(static_cast<OutT*>(p.y) + (OUT ? chunk_base : 0),
                OUT ? static_cast<uint32_t>(steps) * row_out : 0u);
  uint32_t soff_out = 0;
  const InT* Brow = static_cast<const InT*>(p.Bm) + (b * p.L + t0) * N;
  const InT* Crow = static_cast<const InT*>(p.Cm) + (b * p.L + t0) * N;

  float dacc = 0.0f;
  if (steps <= 0) return;

  // Two row buffers used in turn (no register copies): step j computes with
  // buffer j & 1 and fetches the next step's rows into buffer (j + 1) & 1.
  float Bb0[N], Bb1[N], Cb0[N], Cb1[N];
  load_row<N>(Bb0, Brow);
  if constexpr (OUT) load_row<N>(Cb0, Crow);

  auto one_step = [&](float xv, float dv, float zv, bool has_next, float (&Bcur)[N],
                      float (&Bnext)[N], float (&Ccur)[N], float (&Cnext)[N]) {
    // on the last step re-read the current row instead of running past the end
    const int64_t adv = has_next ? N : 0;
    const InT* nb = Brow + adv;
    const InT* nc = Crow + adv;
    // Scalar loads complete out of order, so the only wait for them is "all
    // outstanding".  The next step's rows must therefore be requested after
    // this step's rows have been waited for, or every use of the current row
    // would also wait for the prefetch.  Reading the current rows here (no
    // code is emitted) puts that wait before the two loads below.
    // (Single-state rows may live in VGPRs; they are not worth ordering.)
    constexpr bool kScalarRows = N >= 2;
    if constexpr (kScalarRows && OUT) {
      asm volatile("" : "+s"(nb), "+s"(nc) : "s"(Bcur[0]), "s"(Ccur[0]));
    } else if constexpr (kScalarRows) {
      asm volatile("" : "+s"(nb) : "s"(Bcur[0]));
    }
    load_row<N>(Bnext, nb);
    if constexpr (OUT) load_row<N>(Cnext, nc);
    const float u = CONV ? conv_push(cs, xv) : xv;
    if constexpr (OUT) {
      const float acc = ssm_step_any<N, DISC, true>(h, cc, Bcur, Ccur, u, dv);
      float yv = fmaf(dsk, u, acc);
      if constexpr (GATE) yv *= silu(zv);
      stb(ry, lo_out, soff_out, yv, static_cast<OutT*>(nullptr));
      soff_out += row_out;
    } else {
      ssm_step_any<N, DISC, false, SCALED>(h, cc, Bcur, Bcur, u, dv);
    }
    Brow += N;
    Crow += N;
  };

  // The chunk's sum of Delta feeds exp(A * sum) in the carry combine, so it
  // is kept accurate: block sums of kU steps are added with Kahan
  // compensation (a plain running fp32 sum of a steady Delta drifts by
  // ~length * 2^-25 relative, which the decay amplifies by |A * sum|).
  float dcomp = 0.0f;
  auto sum_add = [&](float v) {
    const float yv = v - dcomp;
    const float tv = dacc + yv;
    dcomp = (tv - dacc) - yv;
    dacc = tv;
  };

  static_assert(kU % 2 == 0, "row buffers alternate within a block");
  const int32_t nblk = steps / kU;
  // SAVE: the state entering step te = t0 + (blk + 1) kU is kept when te is
  // a multiple of kSaveStride below L (chunks start on multiples of kU, so
  // these steps end blocks; the remainder after the last block holds none).
  // The lane's destination row advances in registers; the blocks that save
  // are every kSaveStride / kU-th from save_blk on, below save_lim.
  int32_t save_blk = 0, save_lim = 0;
  float* save_dst = nullptr;
  if constexpr (SAVE) {
    const int64_t first = (t0 / kSaveStride + 1) * kSaveStride;   // first kept step > t0
    save_blk = static_cast<int32_t>((first - t0) / kU) - 1;
    const int64_t lim = (p.L - 1 - t0) / kU;                      // te < L  <=>  blk < lim
    save_lim = static_cast<int32_t>(lim < nblk ? lim : nblk);
    save_dst = p.hsave + ((b * p.nsave + first / kSaveStride - 1) * D + d) * N;
  }
  float xc[kU], dc[kU], zc[kU];
  constexpr InT* kIn = nullptr;
  // byte offset of row t of the chunk, clamped to its last row: rows past the
  // chunk are loaded (so that every path issues the same loads) but never used
  auto row_off = [&](int32_t t) {
    return static_cast<uint32_t>(t < steps ? t : steps - 1) * row_in;
  };
#pragma unroll
  for (int j = 0; j < kU; ++j) {
    xc[j] = ldb(rx, lo_in, row_off(j), kIn);
    dc[j] = ldb(rd, lo_in, row_off(j), kIn);
    zc[j] = GATE ? ldb(rz, lo_in, row_off(j), kIn) : 0.0f;
  }
  for (int32_t blk = 0; blk < nblk; ++blk) {
    // Prefetch the next block's x / Delta (/ z) -- after the last block, the
    // remainder's rows.  The loads are unconditional so that the number of
    // loads in flight is the same on every path and each wait covers only
    // the older loads.
    float xn[kU], dn[kU], zn[kU];
    const int32_t tn = (blk + 1) * kU;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      xn[j] = ldb(rx, lo_in, row_off(tn + j), kIn);
      dn[j] = ldb(rd, lo_in, row_off(tn + j), kIn);
      zn[j] = GATE ? ldb(rz, lo_in, row_off(tn + j), kIn) : 0.0f;
    }
    // the block's step sizes from their pre-activations (wave-uniform branch)
    if (dtm != kDtRaw) {
#pragma unroll
      for (int j = 0; j < kU; ++j) dc[j] = dt_transform(dc[j], dtb, dtm);
    }
    const int32_t tb = blk * kU;
#pragma unroll
    for (int j = 0; j < kU; j += 2) {
      one_step(xc[j], dc[j], zc[j], tb + j + 1 < steps, Bb0, Bb1, Cb0, Cb1);
      one_step(xc[j + 1], dc[j + 1], zc[j + 1], tb + j + 2 < steps, Bb1, Bb0, Cb1, Cb0);
    }
    if constexpr (SAVE) {
      if (blk == save_blk && blk < save_lim) {
#pragma unroll
        for (int n = 0; n < N; ++n) save_dst[n] = h[n];
        save_dst += D * N;
        save_blk += kSaveStride / kU;
      }
    }
    if constexpr (!OUT) {
      float bs = dc[0];
#pragma unroll
      for (int j = 1; j < kU; ++j) bs += dc[j];
      sum_add(bs);
    }
#pragma unroll
    for (int j = 0; j < kU; ++j) { xc[j] = xn[j]; dc[j] = dn[j]; zc[j] = zn[j]; }
  }
  // remainder (fewer than kU steps) from the rows already in registers; the
  // current B / C rows are in Bb0 / Cb0 (every block has an even step count)
  const int32_t rem = steps - nblk * kU;
  if (rem > 0) {
    if (dtm != kDtRaw) {
#pragma unroll
      for (int j = 0; j < kU; ++j) dc[j] = dt_transform(dc[j], dtb, dtm);
    }
    const int32_t tb = nblk * kU;
#pragma unroll
    for (int j = 0; j < kU; j += 2) {
      if (j < rem) {
        one_step(xc[j], dc[j], zc[j], tb + j + 1 < steps, Bb0, Bb1, Cb0, Cb1);
        if constexpr (!OUT) sum_add(dc[j]);
      }
      if (j + 1 < rem) {
        one_step(xc[j + 1], dc[j + 1], zc[j + 1], tb + j + 2 < steps, Bb1, Bb0, Cb1, Cb0);
        if constexpr (!OUT) sum_add(dc[j + 1]);
      }
    }
  }
  if (!OUT && dsum_out) *dsum_out = dacc - dcomp;
  if constexpr (SCALED) {
    // back to h (A is read again rather than kept in registers through the
    // chunk)
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] /= scaled_a(p.A[d * N + n]);
  }
  if constexpr (CONV && OUT) {
    if (cs_save) conv_save(cs, p.conv_k, cs_save);
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Pass 1 (chunked plans): for chunks 0..C-2, the state each chunk reaches from
// a zero state, and its sum of Delta.
// (at most 128 VGPRs, i.e. at least four waves per SIMD, for every variant)
template <int N, typename InT, int DISC, bool CONV>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(4)))
k_chunk_summary(const ScanParams p) {
  const int wg = xcd_remap(blockIdx.x, p.nwg);
  const Tile tl = tile_of(wg, p.dtiles, p.C - 1);
  const int64_t dbase = tl.dtile * kWave;
  const uint32_t lo = lane_offset(dbase, p.D);
  const int64_t d = dbase + lo;
  const int64_t t0 = tl.chunk * p.T;
  const int32_t steps = static_cast<int32_t>(p.T);   // chunks before the last are full
  float h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) h[n] = 0.0f;
  const int64_t slot = tl.b * (p.C - 1) + tl.chunk;
  // (ZOH carries the scaled state A h, see ssm_step_lane)
  chunk_loop<N, InT, float, DISC, CONV, false, false, false, DISC == kZoh>(
      p, tl.b, dbase, lo, t0, steps, h, p.dsum + slot * p.D + d, nullptr);
  float* hs = p.hsum + (slot * p.D + d) * N;
#pragma unroll
  for (int n = 0; n < N; ++n) hs[n] = h[n];
}

// exp(z) * carry + b with z2 = z * log2(e), keeping the decay accurate when
// exp(z) is close to 1: a carry + (r carry + b) with r = exp(z) - a.
__device__ __forceinline__ float decay_add(float z2, float carry, float b) {
  const float a = exp2_fast(z2);
  return fmaf(a, carry, fmaf(exp_residual(z2, a), carry, b));
}

// Exclusive walk over G groups: vals[g] (a group's end state from zero) is
// replaced by the carry into group g, and carry moves past the group.
__device__ __forceinline__ void walk_carry_in(float a2, float carry, const float* sums,
                                              int64_t sstr, float* vals, int64_t vstr, int64_t G) {
  constexpr int U = 8;
  int64_t g = 0;
  for (; g + U <= G; g += U) {
    float sv[U], bv[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      sv[j] = sums[(g + j) * sstr];
      bv[j] = vals[(g + j) * vstr];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      vals[(g + j) * vstr] = carry;
      carry = decay_add(a2 * sv[j], carry, bv[j]);
    }
  }
  for (; g < G; ++g) {
    const float bv = vals[g * vstr];
    vals[g * vstr] = carry;
    carry = decay_add(a2 * sums[g * sstr], carry, bv);
  }
}

// Walk chunks [c0, c1) of one (b, d, n) chain from `carry`:
//   carry <- exp(A * sum_c Delta) * carry + hsum_c
// with the loads of 8 chunks issued before they are folded.  WRITE stores
// each new carry over hsum_c (the carry into chunk c + 1); KAHAN also returns
// the compensated sum of the chunks' Delta sums in *ssum.
template <bool WRITE, bool KAHAN>
__device__ __forceinline__ float walk_chunks(float a2, float carry, const float* ds, int64_t dstr,
                                             float* hs, int64_t hstr, int64_t c0, int64_t c1,
                                             float* ssum) {
  constexpr int U = 8;
  float sacc = 0.0f, scomp = 0.0f;
  auto fold = [&](float sv, float hv, int64_t c) {
    carry = decay_add(a2 * sv, carry, hv);
    if constexpr (WRITE) hs[c * hstr] = carry;
    if constexpr (KAHAN) {
      const float y = sv - scomp;
      const float t = sacc + y;
      scomp = (t - sacc) - y;
      sacc = t;
    }
  };
  int64_t c = c0;
  for (; c + U <= c1; c += U) {
    float sv[U], hv[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      sv[j] = ds[(c + j) * dstr];
      hv[j] = hs[(c + j) * hstr];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) fold(sv[j], hv[j], c + j);
  }
  for (; c < c1; ++c) fold(ds[c * dstr], hs[c * hstr], c);
  if constexpr (KAHAN) *ssum = sacc - scomp;
  return carry;
}

// Pass 2: carries.  One lane per (b, d, n); walks the chunks in order,
//   carry_0 = h0,  carry_{c+1} = exp(A * sum_c Delta) * carry_c + hsum_c,
// and overwrites hsum_c with carry_{c+1}, the carry into chunk c + 1.
template <int N>
__global__ void __launch_bounds__(kWave) k_carry_combine(const ScanParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * DN) return;
  const int64_t b = idx / DN;
  const int64_t dn = idx - b * DN;
  const int64_t d = dn / N;
  const float a2 = p.A[dn] * kLog2e;
  const float carry = p.h0 ? p.h0[idx] : 0.0f;
  const int64_t nc = p.C - 1;
  walk_chunks<true, false>(a2, carry, p.dsum + b * nc * p.D + d, p.D, p.hsum + b * nc * DN + dn,
                           DN, 0, nc, nullptr);
}

// The same carries for long chains, in three parallel steps over groups of
// gsz chunks (the operator is associative, so a group can be folded before
// its carry is known -- 53ai.com explainer, section 3.3):
//   1. per (b, group, d, n): the group's end state from zero and its sum of
//      Delta;
//   2. per (b, d, n): the carry into every group, walking the G groups;
//   3. per (b, group, d, n): the group's chunks again from its carry,
//      writing the carries into hsum.
template <int N>
__global__ void __launch_bounds__(kWave) k_combine_groups(const ScanParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * p.G * DN) return;
  const int64_t bg = idx / DN, dn = idx - bg * DN;
  const int64_t b = bg / p.G, g = bg - b * p.G;
  const int64_t d = dn / N;
  const int64_t nc = p.C - 1;
  const int64_t c0 = g * p.gsz, c1 = (c0 + p.gsz < nc) ? c0 + p.gsz : nc;
  float ssum;
  const float be = walk_chunks<false, true>(p.A[dn] * kLog2e, 0.0f, p.dsum + b * nc * p.D + d,
                                            p.D, p.hsum + b * nc * DN + dn, DN, c0, c1, &ssum);
  p.gB[idx] = be;
  if (dn % N == 0) p.gS[bg * p.D + d] = ssum;
}

template <int N>
__global__ void __launch_bounds__(kWave) k_combine_top(const ScanParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * DN) return;
  const int64_t b = idx / DN, dn = idx - b * DN;
  const int64_t d = dn / N;
  float carry = p.h0 ? p.h0[idx] : 0.0f;
  // gB[g] (the group's end state from zero) becomes the carry into group g
  float* gb = p.gB + b * p.G * DN + dn;
  walk_carry_in(p.A[dn] * kLog2e, carry, p.gS + b * p.G * p.D + d, p.D, gb, DN, p.G);
}

template <int N>
__global__ void __launch_bounds__(kWave) k_combine_apply(const ScanParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
  const int64_t DN = p.D * N;
  if (idx >= p.Bt * p.G * DN) return;
  const int64_t bg = idx / DN, dn = idx - bg * DN;
  const int64_t b = bg / p.G, g = bg - b * p.G;
  const int64_t d = dn / N;
  const int64_t nc = p.C - 1;
  const int64_t c0 = g * p.gsz, c1 = (c0 + p.gsz < nc) ? c0 + p.gsz : nc;
  walk_chunks<true, false>(p.A[dn] * kLog2e, p.gB[idx], p.dsum + b * nc * p.D + d, p.D,
                           p.hsum + b * nc * DN + dn, DN, c0, c1, nullptr);
}

// Pass 3 (or the only pass): scan each chunk from its carry-in, write y, and
// h_last from the final chunk.
template <int N, typename InT, typename OutT, int DISC, bool CONV, bool GATE, bool SAVE>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(4)))
k_scan_out(const ScanParams p) {
  const int wg = xcd_remap(blockIdx.x, p.nwg);
  const Tile tl = tile_of(wg, p.dtiles, p.C);
  const int64_t dbase = tl.dtile * kWave;
  const uint32_t lo = lane_offset(dbase, p.D);
  const int64_t d = dbase + lo;
  const int64_t t0 = tl.chunk * p.T;
  const int32_t steps = static_cast<int32_t>((t0 + p.T < p.L) ? p.T : p.L - t0);
  float h[N];
  if (tl.chunk == 0) {
    if (p.h0) {
      const float* h0 = p.h0 + (tl.b * p.D + d) * N;
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = h0[n];
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = 0.0f;
    }
  } else {
    const float* cin = p.hsum + ((tl.b * (p.C - 1) + tl.chunk - 1) * p.D + d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = cin[n];
  }
  const bool last = tl.chunk == p.C - 1;
  float* cs_save = (CONV && last && p.cs_out && p.conv_k > 1)
                       ? p.cs_out + (tl.b * p.D + d) * (p.conv_k - 1)
                       : nullptr;
  chunk_loop<N, InT, OutT, DISC, CONV, true, GATE, SAVE>(p, tl.b, dbase, lo, t0, steps, h,
                                                         nullptr, cs_save);
  if (p.h_last && last) {
    float* hl = p.h_last + (tl.b * p.D + d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) hl[n] = h[n];
  }
}

// h_last for an empty sequence: a copy of h0 (or zeros).
__global__ void __launch_bounds__(256) k_state_copy(float* dst, const float* src, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// Decode-step lane layout: a channel's N states are split over S = N / NL
// lanes holding NL = min(N, 4) consecutive states each, so a wave covers
// 64 / S channels and every load or store of the state h is one contiguous
// access of the whole wave (1 KB for fp32 with N = 16).  The S partial
// readouts of a channel are summed with quad-lane DPP swaps.
template <int N>
struct StepLayout {
  static constexpr int NL = N < 4 ? N : 4;
  static constexpr int S = N / NL;
  static constexpr int CPW = kWave / S;   // channels per wave
  static constexpr int ROWS = 2;   // batch rows per wave, loaded before any is computed
  static constexpr int WPG = 4;    // waves per workgroup (consecutive channel tiles)
};

__device__ __forceinline__ float dpp_quad_xor1(float v) {
  // quad_perm [1, 0, 3, 2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  // quad_perm [2, 3, 0, 1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// State slices of 4 / 2 / 1 floats as one vector access (the host checks that
// h is aligned to 4 * min(N, 4) bytes).  Both accesses are non-temporal: a
// step reads each state line once and overwrites it, and the next read of
// the line is a whole step (84 MB of state on the decode workload) later.
// Measured on the 256 x 5120 x 16 decode step, against plain accesses: a
// token right after a cache flush 40.5 -> 35.4 us, a 512-token loop 34.0 ->
// 31.4 us (fused steps 48.0 -> 45.5).  Either access alone gains nothing in
// the loop, and non-temporal loads of the token's inputs lost 2 us.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int NL>
__device__ __forceinline__ void load_state(float (&h)[NL], const float* p) {
  if constexpr (NL == 4) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
  } else if constexpr (NL == 2) {
    const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    h[0] = v.x; h[1] = v.y;
  } else {
    h[0] = __builtin_nontemporal_load(p);
  }
}
template <int NL>
__device__ __forceinline__ void store_state(float* p, const float (&h)[NL]) {
  if constexpr (NL == 4) {
    const f32x4 v = {h[0], h[1], h[2], h[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
  } else if constexpr (NL == 2) {
    const f32x2 v = {h[0], h[1]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x2*>(p));
  } else {
    __builtin_nontemporal_store(h[0], p);
  }
}

// Time across the lanes: one wave per channel (b, d), lane i holding step
// t0 + i of a block of 64 steps.  Every lane forms its step's pair
// (Abar, Bbar u) for each state at once, and an inclusive scan over the
// lanes by the associative operator (a, b) o (a', b') = (a a', a' b + b')
// (53ai.com explainer, section 3.3; gsyq.cn deep-dive, 硬件优化并行扫描算法:
// the recurrence evaluated as a tree) leaves in lane i the state that the
// block's steps up to t0 + i reach from a zero state, and the decay product
// over them.  The scan takes six DPP steps across the wave: row_shr 1, 2,
// 4, 8 within each row of 16 lanes, then row_bcast 15 and row_bcast 31
// across rows; a lane whose DPP source lies outside its reach keeps the
// identity (1, 0).  The block's carry-in h then enters as A_i h + b_i, and
// lane 63's state carries into the next block.  A block costs one dependent
// chain of six combines instead of 64 dependent steps, so a short sequence
// of few channels finishes in a fraction of a sequential walk's latency;
// each element costs about six combines of work instead of one step, so the
// plan takes it only for short sequences of few channels, where the chunked
// passes' three launches and their waves' first-step latencies dominate.
//
// Weak decays.  Where some step of the block has |Delta A| below the
// slow-decay threshold (wave-uniform test), each decay is carried as a pair
// a + r, with r the part of exp(Delta A) that rounding a lost
// (exp_residual), and the product of two decays keeps its own rounding
// error, fma(a, a', -a a'), in r.  CONV runs the causal conv prologue per
// lane (each lane loads its step's three earlier inputs) and hands the last
// conv_k - 1 inputs to p.cs_out; GATE multiplies y by silu(z); SAVE writes
// the state entering every kSaveStride-th step to p.hsave.
// One combine of the lane scan: every lane takes the pair of the lane CTRL
// reaches (the identity where it reaches none) as the earlier operand.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_from(float v, float id) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(v), CTRL, ROWS, 0xF, false));
}

template <int CTRL, int ROWS, bool RES, int N>
__device__ __forceinline__ void wave_combine(float (&a)[N], float (&r)[N], float (&bb)[N]) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float ap = dpp_from<CTRL, ROWS>(a[n], 1.0f);
    const float bp = dpp_from<CTRL, ROWS>(bb[n], 0.0f);
    if constexpr (RES) {
      const float rp = dpp_from<CTRL, ROWS>(r[n], 0.0f);
      // (ap + rp, bp) o (a + r, b): b' = (a + r) bp + b, decay (ap + rp)(a + r)
      // with the rounding error of ap a kept in r (rp r is below fp32 resolution)
      bb[n] = fmaf(a[n], bp, fmaf(r[n], bp, bb[n]));
      const float m = ap * a[n];
      r[n] = fmaf(ap, a[n], -m) + fmaf(ap, r[n], rp * a[n]);
      a[n] = m;
    } else {
      bb[n] = fmaf(a[n], bp, bb[n]);
      a[n] = ap * a[n];
    }
  }
}

// Inclusive scan of the pairs over the 64 lanes: row_shr 1, 2, 4, 8 within
// each row of 16 lanes, then row_bcast 15 into rows 1 and 3 and row_bcast 31
// into rows 2 and 3.
template <bool RES, int N>
__device__ __forceinline__ void wave_scan(float (&a)[N], float (&r)[N], float (&bb)[N]) {
  wave_combine<0x111, 0xF, RES>(a, r, bb);
  wave_combine<0x112, 0xF, RES>(a, r, bb);
  wave_combine<0x114, 0xF, RES>(a, r, bb);
  wave_combine<0x118, 0xF, RES>(a, r, bb);
  wave_combine<0x142, 0xA, RES>(a, r, bb);
  wave_combine<0x143, 0xC, RES>(a, r, bb);
}

template <int N, typename InT, typename OutT, int DISC, bool GATE, bool SAVE, bool CONV>
__global__ void __launch_bounds__(kWave) k_scan_wave(const ScanParams p) {
  const int64_t wg = blockIdx.x;
  const int64_t D = p.D, L = p.L;
  const int64_t b = wg / D, d = wg - b * D;
  const int lane = threadIdx.x;
  // conv prologue: the channel's taps (zero-padded at the oldest end) and
  // the caller's window, x[t < 0] = win[S + t] (zero where there is none)
  float cw[kConvTaps] = {0.f, 0.f, 0.f, 0.f};
  float cb = 0.0f;
  const int S = CONV ? p.conv_k - 1 : 0;
  const float* win = (CONV && p.cs_in) ? p.cs_in + (b * D + d) * S : nullptr;
  if constexpr (CONV) {
    for (int k = 0; k < p.conv_k; ++k) cw[kConvTaps - p.conv_k + k] = p.conv_w[d * p.conv_k + k];
    cb = p.conv_b ? p.conv_b[d] : 0.0f;
  }
  ChanConst<N, DISC> cc;
  load_chan<N, DISC>(cc, p.A + d * N, p.exact_thr);
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  const int dtm = p.dt_mode;
  const float dtb = (dtm != kDtRaw && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  const InT* xp = static_cast<const InT*>(p.x) + b * L * D + d;
  const InT* dp = static_cast<const InT*>(p.delta) + b * L * D + d;
  const InT* zp = static_cast<const InT*>(GATE ? p.z : p.x) + b * L * D + d;
  const InT* Bp = static_cast<const InT*>(p.Bm) + b * L * N;
  const InT* Cp = static_cast<const InT*>(p.Cm) + b * L * N;
  OutT* yp = static_cast<OutT*>(p.y) + b * L * D + d;
  float hc[N];   // state entering the block (wave-uniform)
#pragma unroll
  for (int n = 0; n < N; ++n) hc[n] = p.h0 ? p.h0[(b * D + d) * N + n] : 0.0f;
  for (int64_t t0 = 0; t0 < L; t0 += kWave) {
    const int64_t t = t0 + lane;
    const bool in = t < L;
    const int64_t tc = in ? t : L - 1;   // lanes past the end read the last step
    float u = ld(xp + tc * D);
    if constexpr (CONV) {
      // u = silu(bias + sum_k w[k] x[t - 3 + k]): the three earlier inputs
      // from memory (their neighbours' rows, already in cache), or from the
      // window before token 0
      float z = fmaf(cw[3], u, cb);
#pragma unroll
      for (int k = 1; k <= 3; ++k) {
        const int64_t tk = tc - k;
        const float xk = tk >= 0 ? ld(xp + tk * D) : ((win && tk >= -S) ? win[S + tk] : 0.0f);
        z = fmaf(cw[3 - k], xk, z);
      }
      u = silu(z);
    }
    float dv = ld(dp + tc * D);
    if (dtm != kDtRaw) dv = dt_transform(dv, dtb, dtm);
    const float zv = GATE ? ld(zp + tc * D) : 0.0f;
    if (!in) {   // the identity pair: a = exp(0) = 1, b = 0
      u = 0.0f;
      dv = 0.0f;
    }
    float Bv[N], Cv[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      Bv[n] = ld(Bp + tc * N + n);
      Cv[n] = ld(Cp + tc * N + n);
    }
    float h[N];
    // the block's pairs, scanned; RES carries each decay's rounding residual
    auto block = [&](auto form) {
      constexpr bool RES = decltype(form)::value;
      float a[N], r[N], bb[N];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float z2 = dv * cc.A2[n];
        a[n] = exp2_fast(z2);
        r[n] = (RES || DISC == kZoh) ? exp_residual<true>(z2, a[n]) : 0.0f;
        float gu;   // the input factor times u
        if constexpr (DISC == kDeltaB) {
          gu = dv * u;
        } else {
          const float e = (a[n] - 1.0f) + r[n];   // expm1(Delta A)
          gu = (cc.invA[n] != 0.0f) ? (e * cc.invA[n]) * u : dv * u;   // A = 0: limit Delta
        }
        bb[n] = gu * Bv[n];
      }
      wave_scan<RES>(a, r, bb);
#pragma unroll
      for (int n = 0; n < N; ++n)
        h[n] = RES ? fmaf(a[n], hc[n], fmaf(r[n], hc[n], bb[n])) : fmaf(a[n], hc[n], bb[n]);
    };
    if (__builtin_amdgcn_ballot_w64(dv < cc.thr) != 0) block(std::true_type{});
    else block(std::false_type{});
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if (n & 1) acc1 = fmaf(Cv[n], h[n], acc1);
      else acc0 = fmaf(Cv[n], h[n], acc0);
    }
    float yv = fmaf(dsk, u, acc0 + acc1);
    if constexpr (GATE) yv *= silu(zv);
    if (in) st(yp + t * D, yv);
    if constexpr (SAVE) {
      // lane t holds the state entering step t + 1
      if (in && t + 1 < L && (t + 1) % kSaveStride == 0) {
        float* dst = p.hsave + ((b * p.nsave + (t + 1) / kSaveStride - 1) * D + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = h[n];
      }
    }
    if (p.h_last && t == L - 1) {
#pragma unroll
      for (int n = 0; n < N; ++n) p.h_last[(b * D + d) * N + n] = h[n];
    }
#pragma unroll
    for (int n = 0; n < N; ++n)
      hc[n] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h[n]), kWave - 1));
  }
  if constexpr (CONV) {
    // the last S raw inputs, oldest first, reaching into the window when
    // L < S: lane j < S writes x[L - S + j]
    if (p.cs_out && lane < S) {
      const int64_t tj = L - S + lane;
      const float xj = tj >= 0 ? ld(xp + tj * D) : ((win && tj >= -S) ? win[S + tj] : 0.0f);
      p.cs_out[(b * D + d) * S + lane] = xj;
    }
  }
}

// One decode step per sequence, h updated in place.  A wave covers CPW
// channels of ROWS consecutive batch rows (a row past the batch is skipped,
// uniformly for the wave).  Lanes past the last channel duplicate channel
// D - 1: they read the same old state in the same load instruction and store
// identical values.  The optional conv window, step-size transform and gate
// are wave-uniform branches (this kernel is bound by the state traffic).
template <int N, typename InT, typename OutT, int DISC>
__global__ void __launch_bounds__(kWave * StepLayout<N>::WPG) k_step(const StepParams p) {
  constexpr int NL = StepLayout<N>::NL, S = StepLayout<N>::S, CPW = StepLayout<N>::CPW;
  constexpr int ROWS = StepLayout<N>::ROWS, WPG = StepLayout<N>::WPG;
  const int wg = xcd_remap(blockIdx.x, p.nwg);
  const int64_t gtiles = (p.dtiles + WPG - 1) / WPG;
  const int64_t bt = wg / gtiles;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int64_t dtile = (wg - bt * gtiles) * WPG + w;
  // a wave past the last tile exits: a wave duplicating another wave's
  // channels would race with its in-place state update (this kernel has no
  // barrier, so an early exit is safe)
  if (dtile >= p.dtiles) return;
  const int lane = threadIdx.x % kWave;
  const int j = lane % S;
  int64_t d = dtile * CPW + lane / S;
  if (d > p.D - 1) d = p.D - 1;
  const int n0 = j * NL;
  ChanConst<NL, DISC> cc;
  load_chan<NL, DISC>(cc, p.A + d * N + n0, p.exact_thr);
  const float dsk = p.Dskip ? p.Dskip[d] : 0.0f;
  const int dtm = p.dt_mode;
  const float dtb = (dtm != kDtRaw && p.dt_bias) ? p.dt_bias[d] : 0.0f;
  // conv taps, zero-padded at the oldest end as in the scan's prologue
  const int K = p.conv_k;
  const int SW = K > 0 ? K - 1 : 0;   // window length
  float cw[kConvTaps] = {0.f, 0.f, 0.f, 0.f};
  float cb = 0.0f;
  if (K > 0) {
    for (int k = 0; k < K; ++k) cw[kConvTaps - K + k] = p.conv_w[d * K + k];
    cb = p.conv_b ? p.conv_b[d] : 0.0f;
  }
  // Every row's loads are issued before any row is computed or stored (the
  // stores could otherwise alias the next row's loads as far as the compiler
  // knows, and would hold them back): ROWS x 1 KB of state per wave in
  // flight.  Rows past the batch read row Bt - 1 and store nothing.
  float h[ROWS][NL], Bv[ROWS][NL], Cv[ROWS][NL], u[ROWS], dv[ROWS], zg[ROWS];
  float xw[ROWS][3];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    int64_t b = bt * ROWS + r;
    if (b > p.Bt - 1) b = p.Bt - 1;
    load_state<NL>(h[r], p.h + (b * p.D + d) * N + n0);
    const InT* Bp = static_cast<const InT*>(p.Bm) + b * N + n0;
    const InT* Cp = static_cast<const InT*>(p.Cm) + b * N + n0;
#pragma unroll
    for (int n = 0; n < NL; ++n) {
      Bv[r][n] = ld(Bp + n);
      Cv[r][n] = ld(Cp + n);
    }
    u[r] = ld(static_cast<const InT*>(p.x) + b * p.D + d);
    dv[r] = ld(static_cast<const InT*>(p.delta) + b * p.D + d);
    zg[r] = p.z ? ld(static_cast<const InT*>(p.z) + b * p.D + d) : 0.0f;
    if (K > 0) {
      // window x[-SW .. -1] (oldest first) as x[-3], x[-2], x[-1] (zero
      // where the window is shorter); three independent loads
      const float* win = p.conv_state + (b * p.D + d) * SW;
      xw[r][0] = SW >= 3 ? win[SW - 3] : 0.0f;
      xw[r][1] = SW >= 2 ? win[SW - 2] : 0.0f;
      xw[r][2] = SW >= 1 ? win[SW - 1] : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int64_t b = bt * ROWS + r;
    if (b >= p.Bt) break;
    float ur = u[r];
    float dvr = dv[r];
    if (dtm != kDtRaw) dvr = dt_transform(dvr, dtb, dtm);
    if (K > 0) {
      float zc = fmaf(cw[3], ur, cb);
      zc = fmaf(cw[2], xw[r][2], zc);
      zc = fmaf(cw[1], xw[r][1], zc);
      zc = fmaf(cw[0], xw[r][0], zc);
      // the window moves on by one input (written by one lane per channel;
      // every lane of the wave read it above)
      if (j == 0) {
        float* win = p.conv_state + (b * p.D + d) * SW;
        if (SW >= 3) win[SW - 3] = xw[r][1];
        if (SW >= 2) win[SW - 2] = xw[r][2];
        if (SW >= 1) win[SW - 1] = ur;
      }
      ur = silu(zc);
    }
    float acc = ssm_step_any<NL, DISC, true>(h[r], cc, Bv[r], Cv[r], ur, dvr);
    if constexpr (S >= 2) acc += dpp_quad_xor1(acc);
    if constexpr (S >= 4) acc += dpp_quad_xor2(acc);
    store_state<NL>(p.h + (b * p.D + d) * N + n0, h[r]);
    if (j == 0) {
      float yv = fmaf(dsk, ur, acc);
      if (p.z) yv *= silu(zg[r]);
      st(static_cast<OutT*>(p.y) + b * p.D + d, yv);
    }
  }
}

}  // namespace ssmk
