// ssm_scan.hip -- host side of libssmscan.so: argument checks, the chunk plan,
// template dispatch and kernel launches.  The device code is ssm_kernels.hpp;
// the public contract is include/ssm_scan.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "ssm_scan.h"
#include "ssm_kernels.hpp"
#include "ssm_bwd.hpp"

// Device scratch of the allocation-free forward entry point
// (ssm_scan_fwd_noalloc): the chunk summaries, carries and group carries that
// ssm_scan_fwd keeps in the caller's workspace.  One copy per GPU, held
// until the process ends.  Host code never uses this name as an address: the
// per-device address comes from hipGetSymbolAddress.
constexpr size_t kNoallocScratchBytes = size_t(SSM_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local char g_msg[512] = "";

ssm_status_t fail(ssm_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

// The plan targets MI355X: 256 CUs x 4 SIMDs, and scan kernels small enough
// for four waves per SIMD.  A chunked plan uses at most kTargetWaves waves in
// the output pass (rounding the chunk count down, so no partial extra round
// of waves forms a tail), and never cuts chunks shorter than kMinChunk steps.
// Problems too small to fill the chip gain most from short chunks: one wave
// walking a long chunk alone is latency-bound (measured: 1 x 256 x 64 x 16,
// 68.7 us at 64-step chunks, 18.9 us at 8; 2 x 2048 x 64 x 16, 72.5 vs
// 26.5 us; 4-step chunks lost again on the latter).
// Where four waves per SIMD would cut chunks shorter than kShortChunk steps,
// the plan takes three per SIMD instead (kShortTargetWaves): each wave's
// start (its carry, constants and first rows) is then paid by fewer, longer
// chunks.  Measured on fp32 inputs: 4 x 2048 x 768 x 16, 28-step chunks
// (3,552 waves) 63 us vs 32-step chunks (3,072 waves) 53 us; 8 x 4096 x
// 384 x 16, 52 vs 64 steps, 93 vs 84 us.  At 64 steps and more, three and
// four waves per SIMD measured the same or four better (the bench workloads
// keep their plans).
// Where the wave target already cuts the sequence into kBalanceChunks or
// more chunks, chunks are also capped at kLongChunk steps.  The summary pass
// then covers at least 15/16 of the elements anyway, so more chunks add
// little work, while many shorter waves let the dispatcher even out the
// SIMDs: 4096 waves of thousands of steps each cannot.  Measured on
// 1 x 2^20 x 512 x 16 bf16 (whole scan): 2048-step chunks 2.87 ms, 1024
// 2.61, 512 2.52, 256 2.50, 128 2.60; 4 x 8192 x 2560 x 16 bf16 with ZOH and
// the conv: 328 steps 677 us, 256 steps 661 us.
// Sequences of at most kNoSplitSteps steps are not cut at all: the summary
// and carry launches cost more than a wave walking the few steps saves.
// Measured, fp32, us per call back to back (one chunk / 8-step chunks):
// 1 x 16 x 2048 x 16 6.6 / 11.6; 1 x 16 x 4096 x 16 with the conv 8.1 /
// 13.5; 1 x 32 x 4096 x 16 10.7 / 12.7, with the conv 12.4 / 14.5.
constexpr int64_t kNoSplitSteps = 32;
constexpr int64_t kTargetWaves = 4096;
constexpr int64_t kShortTargetWaves = 3072;
constexpr int64_t kShortChunk = 64;
constexpr int64_t kBalanceChunks = 16;
constexpr int64_t kLongChunk = 256;
constexpr int64_t kMinChunk = 8;
constexpr int64_t kChunkAlign = 4;
constexpr int64_t kMaxChunk = int64_t(1) << 30;   // kernels count steps in 32 bits
// A chunk's rows of x / Delta / y are addressed through one buffer resource
// with 32-bit offsets: keep steps * D * 4 bytes below 2^31.
constexpr int64_t kMaxChunkBytes = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

size_t dtype_size(int32_t dt) { return dt == SSM_BF16 ? 2 : 4; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool supported_n(int64_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

// States kept for the backward pass: those entering steps 16, 32, ... < L.
int64_t saved_count(int64_t L) {
  return L > 0 ? (L + ssmk::kSaveStride - 1) / ssmk::kSaveStride - 1 : 0;
}

// A carry walk over more than kGroupWalk chunks is done in groups (three
// parallel steps instead of one sequential chain per (b, d, n)) when it has
// fewer than kGroupChains chains.  With that many chains the sequential walk
// already streams the summaries at HBM speed, and grouping would only read
// them twice (measured: 8 x 2048 x 1536 x 16 backward, 128 fine chunks,
// 717 us sequential vs 757 us grouped; 1 x 2^20 x 512 x 16, 8192 chains,
// 14.8 ms grouped vs 19.0 ms sequential).
constexpr int64_t kGroupWalk = 64;
constexpr int64_t kGroupChains = 65536;
constexpr int64_t kBwdShortChunk = 128;   // backward super-chunk length, see make_bwd_plan
constexpr int64_t kBwdLongChunk = 512;    // backward super-chunk length, see make_bwd_plan

struct Grouping {
  int64_t G = 0, gsz = 0;   // groups of gsz chunks (G = 0: one sequential walk)
};

Grouping grouping(int64_t nc, int64_t chains) {
  Grouping g;
  if (nc <= kGroupWalk || chains >= kGroupChains) return g;
  int64_t G = 1;
  while (G * G < nc) ++G;
  g.gsz = (nc + G - 1) / G;
  g.G = (nc + g.gsz - 1) / g.gsz;
  return g;
}

struct Plan {
  bool wave = false;   // one pass, lanes over time steps, a DPP scan per block (k_scan_wave); C = 1
  int64_t T = 0;       // chunk length
  int64_t C = 0;       // chunks
  int64_t dtiles = 0;  // ceil(D / 64)
  Grouping grp;        // of the carry walk
  size_t ws_dsum = 0;  // bytes
  size_t ws_hsum = 0;
  size_t ws_gS = 0, ws_gB = 0;
  size_t ws_total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Sizes are assumed validated (non-negative, no overflow).
Plan make_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, int32_t chunk_len) {
  Plan pl;
  pl.dtiles = (D + ssmk::kWave - 1) / ssmk::kWave;
  if (L == 0 || Bt * D == 0) return pl;
  int64_t T;
  if (chunk_len > 0) {
    T = std::min<int64_t>(chunk_len, L);
  } else {
    const int64_t waves = Bt * pl.dtiles;
    auto chunks = [&](int64_t target) {
      return std::max<int64_t>(1, std::min<int64_t>(target / waves, L / kMinChunk));
    };
    int64_t C = chunks(kTargetWaves);
    if (C > 1 && (L + C - 1) / C < kShortChunk) C = chunks(kShortTargetWaves);
    if (L <= kNoSplitSteps) C = 1;
    T = (L + C - 1) / C;
    if (C > 1) T = (T + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    if (C >= kBalanceChunks) T = std::min(T, kLongChunk);
    T = std::min(T, L);
  }
  pl.T = std::min({T, kMaxChunk, std::max<int64_t>(1, kMaxChunkBytes / (D * 4))});
  pl.C = (L + pl.T - 1) / pl.T;
  if (pl.C > 1) {
    pl.ws_dsum = align256(size_t(Bt) * size_t(pl.C - 1) * size_t(D) * 4);
    pl.ws_hsum = align256(size_t(Bt) * size_t(pl.C - 1) * size_t(D) * size_t(N) * 4);
    pl.grp = grouping(pl.C - 1, Bt * D * N);
    pl.ws_gS = align256(size_t(Bt) * size_t(pl.grp.G) * size_t(D) * 4);
    pl.ws_gB = align256(size_t(Bt) * size_t(pl.grp.G) * size_t(D) * size_t(N) * 4);
    pl.ws_total = pl.ws_dsum + pl.ws_hsum + pl.ws_gS + pl.ws_gB;
  }
  return pl;
}

// Whether a problem takes the one-pass lane scan (k_scan_wave: time steps
// across a wave's lanes, one wave per channel, a DPP scan per block of 64
// steps, the conv prologue per lane): no forced chunk length, and a short
// sequence of few channels.  A block's six
// dependent combines take about 1.5 us alone on a SIMD, and every element
// costs about six combines of work instead of one recurrence step, so it
// wins where the chunked plan's three launches and its waves' first-step
// latencies dominate: at most 8 blocks (seqlen <= 512) and at most 4096
// wave-blocks (batch * dim * ceil(seqlen / 64)), or 64 * seqlen of them for
// sequences shorter than a block, whose lanes stand partly idle while the
// chunked plan walks the few steps in one chunk (fp32, us per call, lane
// scan / one chunk: 1 x 8 x 256 x 16 6.2 / 6.3, 1 x 8 x 2048 x 16 7.5 /
// 6.2, 1 x 16 x 2048 x 16 7.6 / 6.6, 1 x 32 x 2048 x 16 8.1 / 10.6,
// 2 x 32 x 2048 x 16 12.3 / 10.7, with the conv alike).  Measured, us per call
// back to back (chunked passes / lane scan): 1 x 128 x 256 x 16 bf16
// 14.8 / 6.0; 2 x 256 x 128 x 16 fp32 15.8 / 9.0;
// 4 x 64 x 1024 x 16 fp32 12.4 / 9.6; 1 x 512 x 32 x 16 fp32 17.8 / 14.7;
// 4 x 128 x 256 x 16 bf16 ZOH 17.2 / 8.5; but 1 x 1024 x 32 x 16 fp32
// 19.6 / 27.2, 8 x 128 x 1024 x 16 fp32 ZOH 39.6 / 44.9 and
// 16 x 64 x 2560 x 16 bf16 36.1 / 56.4.
constexpr int64_t kWaveMaxSteps = 512;
constexpr int64_t kWaveMaxBlocks = 4096;
bool wave_wins(int64_t Bt, int64_t L, int64_t D) {
  const int64_t blocks = (L + ssmk::kWave - 1) / ssmk::kWave;
  return L <= kWaveMaxSteps && Bt * D <= std::min(kWaveMaxBlocks, ssmk::kWave * L) / blocks;
}

Plan one_pass_plan(const ssm_scan_args_t* a, const Plan& chunked) {
  const int64_t L = a->seqlen, D = a->dim;
  if (a->chunk_len > 0 || L == 0 || a->batch * D == 0) return chunked;
  if (!wave_wins(a->batch, L, D)) return chunked;
  Plan pl;
  pl.wave = true;
  pl.T = L;
  pl.C = 1;
  pl.dtiles = chunked.dtiles;
  return pl;
}

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool misaligned(const void* p, size_t align) {
  return p && (reinterpret_cast<uintptr_t>(p) % align) != 0;
}

// The plan of the allocation-free entry point: the library's plan when its
// summaries fit the scratch array, otherwise the same plan with chunks
// lengthened (by doubling, kept a multiple of 4) until they do; a chunk
// length the caller forces is kept as given.
Plan scratch_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, int32_t chunk_len) {
  Plan pl = make_plan(Bt, L, D, N, chunk_len);
  if (chunk_len > 0) return pl;
  while (pl.ws_total > kNoallocScratchBytes && pl.C > 1) {
    int64_t T = std::min<int64_t>(L, (2 * pl.T + kChunkAlign - 1) / kChunkAlign * kChunkAlign);
    if (T > INT32_MAX) T = L;
    const Plan next = make_plan(Bt, L, D, N, static_cast<int32_t>(std::min<int64_t>(T, INT32_MAX)));
    if (next.T <= pl.T) break;   // capped (32-bit row offsets): cannot lengthen further
    pl = next;
  }
  return pl;
}

// Validation common to the scan; fills the plan on success.  With
// `own_scratch` (the allocation-free entry point) the plan must fit the
// library's scratch array, and the caller's workspace fields are ignored.
ssm_status_t check_scan(const ssm_scan_args_t* a, Plan* plan, bool own_scratch = false) {
  if (!a) return fail(SSM_ERR_NULL, "args is NULL");
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 0)
    return fail(SSM_ERR_SHAPE, "negative size: batch=%lld seqlen=%lld dim=%lld",
                (long long)a->batch, (long long)a->seqlen, (long long)a->dim);
  if (a->dstate < 1) return fail(SSM_ERR_SHAPE, "dstate must be >= 1 (got %lld)", (long long)a->dstate);
  if (a->in_dtype != SSM_F32 && a->in_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "unknown in_dtype %d", a->in_dtype);
  if (a->out_dtype != SSM_F32 && a->out_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "unknown out_dtype %d", a->out_dtype);
  if (a->disc != SSM_DISC_DELTA_B && a->disc != SSM_DISC_ZOH)
    return fail(SSM_ERR_DTYPE, "unknown discretization %d", a->disc);
  if (!supported_n(a->dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {1,2,4,8,16}", (long long)a->dstate);
  if (a->conv_w && (a->conv_k < 1 || a->conv_k > ssmk::kConvTaps))
    return fail(SSM_ERR_UNSUPPORTED, "conv_k %d not in 1..4", a->conv_k);
  if (a->chunk_len < 0) return fail(SSM_ERR_UNSUPPORTED, "chunk_len must be >= 0");
  if (a->reserved != 0 || a->reserved2 != 0)
    return fail(SSM_ERR_UNSUPPORTED, "reserved fields must be 0");
  if (a->delta_softplus != 0 && a->delta_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
  if (!a->conv_w && (a->conv_state_in || a->conv_state_out))
    return fail(SSM_ERR_UNSUPPORTED, "conv_state_in / conv_state_out need conv_w");
  // byte counts must fit in int64 (and the grid in a launch)
  int64_t bl, bld, bln, dn, bdn, bds;
  const int64_t win = a->conv_w ? a->conv_k - 1 : 0;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) ||
      !mul_ok(bl, a->dstate, &bln) || !mul_ok(a->dim, a->dstate, &dn) ||
      !mul_ok(a->batch, dn, &bdn) || bld > INT64_MAX / 8 || bln > INT64_MAX / 8 ||
      bdn > INT64_MAX / 8 || !mul_ok(a->batch * a->dim, win, &bds) || bds > INT64_MAX / 8)
    return fail(SSM_ERR_SHAPE, "sizes overflow");
  *plan = one_pass_plan(a, own_scratch
                           ? scratch_plan(a->batch, a->seqlen, a->dim, a->dstate, a->chunk_len)
                           : make_plan(a->batch, a->seqlen, a->dim, a->dstate, a->chunk_len));
  if (own_scratch && plan->ws_total > kNoallocScratchBytes)
    return fail(SSM_ERR_WORKSPACE,
                "the chunk summaries of this plan need %zu bytes of scratch; the "
                "allocation-free entry point holds %zu (pass chunk_len = 0, or a longer one)",
                plan->ws_total, kNoallocScratchBytes);
  const Range cso{win > 0 ? a->conv_state_out : nullptr, size_t(bds) * 4};
  const Range csi{win > 0 ? a->conv_state_in : nullptr, size_t(bds) * 4};
  if (misaligned(a->conv_state_in, 4) || misaligned(a->conv_state_out, 4))
    return fail(SSM_ERR_UNSUPPORTED, "misaligned conv state (4 bytes)");
  // kept states: the output pass writes them at block ends, which fall on
  // multiples of 16 only when chunks start on multiples of 4
  const int64_t nsave = saved_count(a->seqlen);
  const Range hsv{nsave > 0 ? a->h_saved : nullptr, size_t(bdn) * size_t(nsave) * 4};
  if (misaligned(a->h_saved, 4)) return fail(SSM_ERR_UNSUPPORTED, "misaligned h_saved (4 bytes)");
  if (hsv.p && plan->C > 1 && plan->T % ssmk::kUnrollOut != 0)
    return fail(SSM_ERR_UNSUPPORTED, "h_saved needs a chunk length that is a multiple of %d "
                "(got %lld)", ssmk::kUnrollOut, (long long)plan->T);
  if (a->seqlen == 0 || a->batch * a->dim == 0) {
    // only h_last (with h0 or zeros) and conv_state_out (with conv_state_in or
    // zeros) may be written
    if (a->batch * a->dim > 0) {
      const Range hl{a->h_last, size_t(bdn) * 4}, h0{a->h0, size_t(bdn) * 4};
      if (overlap(hl, h0) || overlap(hl, csi) || overlap(hl, cso) || overlap(cso, csi) ||
          overlap(cso, h0))
        return fail(SSM_ERR_ALIAS, "an output overlaps another buffer");
    }
    return SSM_OK;
  }
  if (!a->x || !a->delta || !a->A || !a->Bm || !a->Cm || !a->y)
    return fail(SSM_ERR_NULL, "x, delta, A, Bm, Cm and y are required");
  const size_t in_sz = dtype_size(a->in_dtype), out_sz = dtype_size(a->out_dtype);
  if (misaligned(a->x, in_sz) || misaligned(a->delta, in_sz) || misaligned(a->Bm, 4) ||
      misaligned(a->Cm, 4) || misaligned(a->y, out_sz) || misaligned(a->A, 4) ||
      misaligned(a->Dskip, 4) || misaligned(a->h0, 4) || misaligned(a->h_last, 4) ||
      misaligned(a->conv_w, 4) || misaligned(a->conv_b, 4) || misaligned(a->workspace, 256) ||
      misaligned(a->z, in_sz) || misaligned(a->delta_bias, 4))
    return fail(SSM_ERR_UNSUPPORTED,
                "misaligned pointer (element alignment; B, C 4 bytes; workspace 256 bytes)");
  const Range y{a->y, size_t(bld) * out_sz};
  const Range hl{a->h_last, size_t(bdn) * 4};
  const Range ins[] = {
      {a->x, size_t(bld) * in_sz},        {a->delta, size_t(bld) * in_sz},
      {a->A, size_t(dn) * 4},             {a->Bm, size_t(bln) * in_sz},
      {a->Cm, size_t(bln) * in_sz},       {a->Dskip, size_t(a->dim) * 4},
      {a->h0, size_t(bdn) * 4},           {a->conv_w, size_t(a->dim) * size_t(std::max(a->conv_k, 0)) * 4},
      {a->conv_b, a->conv_w ? size_t(a->dim) * 4 : 0},
      {a->delta_bias, size_t(a->dim) * 4}, {a->z, size_t(bld) * in_sz},
      csi,
  };
  for (const Range& r : ins) {
    if (overlap(y, r)) return fail(SSM_ERR_ALIAS, "y overlaps an input");
    if (overlap(hl, r)) return fail(SSM_ERR_ALIAS, "h_last overlaps an input");
    if (overlap(cso, r)) return fail(SSM_ERR_ALIAS, "conv_state_out overlaps an input");
    if (overlap(hsv, r)) return fail(SSM_ERR_ALIAS, "h_saved overlaps an input");
  }
  if (overlap(y, hl)) return fail(SSM_ERR_ALIAS, "y overlaps h_last");
  if (overlap(y, cso) || overlap(hl, cso))
    return fail(SSM_ERR_ALIAS, "conv_state_out overlaps an output");
  if (overlap(hsv, y) || overlap(hsv, hl) || overlap(hsv, cso))
    return fail(SSM_ERR_ALIAS, "h_saved overlaps an output");
  if (plan->ws_total > 0 && !own_scratch) {
    if (!a->workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", plan->ws_total);
    if (a->workspace_bytes < plan->ws_total)
      return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", a->workspace_bytes,
                  plan->ws_total);
    const Range ws{a->workspace, plan->ws_total};
    for (const Range& r : ins)
      if (overlap(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps an input");
    if (overlap(ws, y) || overlap(ws, hl) || overlap(ws, cso) || overlap(ws, hsv))
      return fail(SSM_ERR_ALIAS, "workspace overlaps an output");
  }
  const int64_t grid_out = a->batch * plan->C * plan->dtiles;
  const int64_t walk_lanes = a->batch * a->dim * a->dstate * std::max<int64_t>(1, plan->grp.G);
  if (grid_out > kMaxGrid || (walk_lanes + 63) / 64 > kMaxGrid)
    return fail(SSM_ERR_SHAPE, "problem too large for one launch");
  return SSM_OK;
}

ssm_status_t check_step(const ssm_step_args_t* a) {
  if (!a) return fail(SSM_ERR_NULL, "args is NULL");
  if (a->batch < 0 || a->dim < 0)
    return fail(SSM_ERR_SHAPE, "negative size: batch=%lld dim=%lld", (long long)a->batch,
                (long long)a->dim);
  if (a->dstate < 1) return fail(SSM_ERR_SHAPE, "dstate must be >= 1 (got %lld)", (long long)a->dstate);
  if (a->in_dtype != SSM_F32 && a->in_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "unknown in_dtype %d", a->in_dtype);
  if (a->out_dtype != SSM_F32 && a->out_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "unknown out_dtype %d", a->out_dtype);
  if (a->disc != SSM_DISC_DELTA_B && a->disc != SSM_DISC_ZOH)
    return fail(SSM_ERR_DTYPE, "unknown discretization %d", a->disc);
  if (!supported_n(a->dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {1,2,4,8,16}", (long long)a->dstate);
  if (a->reserved != 0) return fail(SSM_ERR_UNSUPPORTED, "reserved field must be 0");
  if (a->delta_softplus != 0 && a->delta_softplus != 1)
    return fail(SSM_ERR_UNSUPPORTED, "delta_softplus must be 0 or 1");
  if (a->conv_w && (a->conv_k < 1 || a->conv_k > ssmk::kConvTaps))
    return fail(SSM_ERR_UNSUPPORTED, "conv_k %d not in 1..4", a->conv_k);
  const int64_t win = a->conv_w ? a->conv_k - 1 : 0;
  int64_t bd, dn, bdn, bn, bds;
  if (!mul_ok(a->batch, a->dim, &bd) || !mul_ok(a->dim, a->dstate, &dn) ||
      !mul_ok(a->batch, dn, &bdn) || !mul_ok(a->batch, a->dstate, &bn) || bdn > INT64_MAX / 8 ||
      !mul_ok(bd, win, &bds) || bds > INT64_MAX / 8)
    return fail(SSM_ERR_SHAPE, "sizes overflow");
  if (bd == 0) return SSM_OK;
  if (!a->x || !a->delta || !a->A || !a->Bm || !a->Cm || !a->h || !a->y)
    return fail(SSM_ERR_NULL, "x, delta, A, Bm, Cm, h and y are required");
  if (win > 0 && !a->conv_state)
    return fail(SSM_ERR_NULL, "conv_state is required with a conv of more than one tap");
  const size_t in_sz = dtype_size(a->in_dtype), out_sz = dtype_size(a->out_dtype);
  if (misaligned(a->x, in_sz) || misaligned(a->delta, in_sz) || misaligned(a->Bm, 4) ||
      misaligned(a->Cm, 4) || misaligned(a->y, out_sz) || misaligned(a->A, 4) ||
      misaligned(a->Dskip, 4) || misaligned(a->h, 4 * size_t(std::min<int64_t>(a->dstate, 4))) ||
      misaligned(a->z, in_sz) || misaligned(a->delta_bias, 4) || misaligned(a->conv_w, 4) ||
      misaligned(a->conv_b, 4) || misaligned(a->conv_state, 4))
    return fail(SSM_ERR_UNSUPPORTED,
                "misaligned pointer (element alignment; B, C 4 bytes; h 4 * min(N, 4) bytes)");
  const Range y{a->y, size_t(bd) * out_sz};
  const Range h{a->h, size_t(bdn) * 4};
  const Range cs{win > 0 ? a->conv_state : nullptr, size_t(bds) * 4};
  const Range ins[] = {{a->x, size_t(bd) * in_sz},     {a->delta, size_t(bd) * in_sz},
                       {a->A, size_t(dn) * 4},         {a->Bm, size_t(bn) * in_sz},
                       {a->Cm, size_t(bn) * in_sz},    {a->Dskip, size_t(a->dim) * 4},
                       {a->z, size_t(bd) * in_sz},     {a->delta_bias, size_t(a->dim) * 4},
                       {a->conv_w, a->conv_w ? size_t(a->dim) * size_t(a->conv_k) * 4 : 0},
                       {a->conv_b, a->conv_w ? size_t(a->dim) * 4 : 0}};
  for (const Range& r : ins) {
    if (overlap(y, r)) return fail(SSM_ERR_ALIAS, "y overlaps an input");
    if (overlap(h, r)) return fail(SSM_ERR_ALIAS, "h overlaps an input");
    if (overlap(cs, r)) return fail(SSM_ERR_ALIAS, "conv_state overlaps an input");
  }
  if (overlap(y, h)) return fail(SSM_ERR_ALIAS, "y overlaps h");
  if (overlap(y, cs) || overlap(h, cs)) return fail(SSM_ERR_ALIAS, "conv_state overlaps an output");
  if ((a->batch * ((a->dim + 15) / 16)) > kMaxGrid) return fail(SSM_ERR_SHAPE, "problem too large");
  return SSM_OK;
}

// A step where some lane has min_n |Delta A[n]| below this threshold runs
// the slow-decay form (Abar plus its rounding residual, from the expm1
// series of Delta A) instead of the fast one.  The fast
// form's error is about 2^-24 / |Delta A| relative: on the decay rate for
// Delta*B, and additionally on the input term for ZOH ((a - 1) / A).  The
// thresholds keep that well inside the tolerance of each input precision.
float exact_threshold(int32_t disc, int32_t in_dtype) {
  if (disc == SSM_DISC_ZOH) return in_dtype == SSM_BF16 ? 1.0f / 8192.0f : 0.03f;
  return in_dtype == SSM_BF16 ? 1.0f / 8192.0f : 1.0f / 1024.0f;
}

// Per-device address of `scratch`, looked up with that device current on the
// first allocation-free call that needs it.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ssm_status_t scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SSM_ERR_UNSUPPORTED, "device %d", dev);
  if (s) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(SSM_ERR_UNSUPPORTED,
                  "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSM_OK;
}

ssm_status_t launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SSM_OK;
}

// The carry walk of pass 2: kp.dsum / kp.hsum hold C - 1 chunk summaries;
// with a grouping, kp.gS / kp.gB must point at the group buffers.
template <int N>
ssm_status_t launch_combine(ssmk::ScanParams kp, const Grouping& grp, hipStream_t s) {
  const int64_t chains = kp.Bt * kp.D * N;
  if (grp.G == 0) {
    hipLaunchKernelGGL((ssmk::k_carry_combine<N>), dim3(uint32_t((chains + 63) / 64)),
                       dim3(ssmk::kWave), 0, s, kp);
    return launch_status("k_carry_combine");
  }
  kp.G = grp.G;
  kp.gsz = grp.gsz;
  const int64_t lanes = chains * grp.G;
  hipLaunchKernelGGL((ssmk::k_combine_groups<N>), dim3(uint32_t((lanes + 63) / 64)),
                     dim3(ssmk::kWave), 0, s, kp);
  if (ssm_status_t st = launch_status("k_combine_groups")) return st;
  hipLaunchKernelGGL((ssmk::k_combine_top<N>), dim3(uint32_t((chains + 63) / 64)),
                     dim3(ssmk::kWave), 0, s, kp);
  if (ssm_status_t st = launch_status("k_combine_top")) return st;
  hipLaunchKernelGGL((ssmk::k_combine_apply<N>), dim3(uint32_t((lanes + 63) / 64)),
                     dim3(ssmk::kWave), 0, s, kp);
  return launch_status("k_combine_apply");
}

template <int N, typename InT, typename OutT, int DISC, bool CONV, bool GATE>
ssm_status_t run_scan(ssmk::ScanParams kp, const Plan& pl, hipStream_t s, hipEvent_t ev0,
                      hipEvent_t ev1) {
  if (pl.wave) {
    kp.nwg = int32_t(kp.Bt * kp.D);
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return fail(SSM_ERR_HIP, "hipEventRecord failed");
    if (kp.hsave)
      hipLaunchKernelGGL((ssmk::k_scan_wave<N, InT, OutT, DISC, GATE, true, CONV>), dim3(kp.nwg),
                         dim3(ssmk::kWave), 0, s, kp);
    else
      hipLaunchKernelGGL((ssmk::k_scan_wave<N, InT, OutT, DISC, GATE, false, CONV>), dim3(kp.nwg),
                         dim3(ssmk::kWave), 0, s, kp);
    if (ssm_status_t st = launch_status("k_scan_wave")) return st;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return fail(SSM_ERR_HIP, "hipEventRecord failed");
    return SSM_OK;
  }
  if (pl.C > 1) {
    kp.nwg = int32_t(kp.Bt * (pl.C - 1) * pl.dtiles);
    hipLaunchKernelGGL((ssmk::k_chunk_summary<N, InT, DISC, CONV>), dim3(kp.nwg), dim3(ssmk::kWave),
                       0, s, kp);
    if (ssm_status_t st = launch_status("k_chunk_summary")) return st;
    if (ssm_status_t st = launch_combine<N>(kp, pl.grp, s)) return st;
  }
  kp.nwg = int32_t(kp.Bt * pl.C * pl.dtiles);
  if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return fail(SSM_ERR_HIP, "hipEventRecord failed");
  if (kp.hsave)
    hipLaunchKernelGGL((ssmk::k_scan_out<N, InT, OutT, DISC, CONV, GATE, true>), dim3(kp.nwg),
                       dim3(ssmk::kWave), 0, s, kp);
  else
    hipLaunchKernelGGL((ssmk::k_scan_out<N, InT, OutT, DISC, CONV, GATE, false>), dim3(kp.nwg),
                       dim3(ssmk::kWave), 0, s, kp);
  if (ssm_status_t st = launch_status("k_scan_out")) return st;
  if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return fail(SSM_ERR_HIP, "hipEventRecord failed");
  return SSM_OK;
}

template <int N, typename InT, typename OutT>
ssm_status_t dispatch_disc(const ssm_scan_args_t* a, const ssmk::ScanParams& kp, const Plan& pl,
                           hipStream_t s) {
  hipEvent_t e0 = static_cast<hipEvent_t>(a->ev_main_start);
  hipEvent_t e1 = static_cast<hipEvent_t>(a->ev_main_stop);
  const bool conv = a->conv_w != nullptr;
  const bool gate = a->z != nullptr;
  using namespace ssmk;
  if (a->disc == SSM_DISC_ZOH) {
    if (gate)
      return conv ? run_scan<N, InT, OutT, kZoh, true, true>(kp, pl, s, e0, e1)
                  : run_scan<N, InT, OutT, kZoh, false, true>(kp, pl, s, e0, e1);
    return conv ? run_scan<N, InT, OutT, kZoh, true, false>(kp, pl, s, e0, e1)
                : run_scan<N, InT, OutT, kZoh, false, false>(kp, pl, s, e0, e1);
  }
  if (gate)
    return conv ? run_scan<N, InT, OutT, kDeltaB, true, true>(kp, pl, s, e0, e1)
                : run_scan<N, InT, OutT, kDeltaB, false, true>(kp, pl, s, e0, e1);
  return conv ? run_scan<N, InT, OutT, kDeltaB, true, false>(kp, pl, s, e0, e1)
              : run_scan<N, InT, OutT, kDeltaB, false, false>(kp, pl, s, e0, e1);
}

int32_t dt_mode_of(const float* bias, int32_t softplus) {
  if (softplus) return ssmk::kDtSoftplus;
  return bias ? ssmk::kDtBias : ssmk::kDtRaw;
}

template <int N>
ssm_status_t dispatch_types(const ssm_scan_args_t* a, const ssmk::ScanParams& kp, const Plan& pl,
                            hipStream_t s) {
  using ssmk::bf16_t;
  if (a->in_dtype == SSM_F32)
    return a->out_dtype == SSM_F32 ? dispatch_disc<N, float, float>(a, kp, pl, s)
                                   : dispatch_disc<N, float, bf16_t>(a, kp, pl, s);
  return a->out_dtype == SSM_F32 ? dispatch_disc<N, bf16_t, float>(a, kp, pl, s)
                                 : dispatch_disc<N, bf16_t, bf16_t>(a, kp, pl, s);
}

template <int N, typename InT, typename OutT>
ssm_status_t run_step_t(const ssm_step_args_t* a, ssmk::StepParams kp, hipStream_t s) {
  constexpr int cpw = ssmk::StepLayout<N>::CPW;
  constexpr int rows = ssmk::StepLayout<N>::ROWS, wpg = ssmk::StepLayout<N>::WPG;
  kp.dtiles = int32_t((a->dim + cpw - 1) / cpw);
  kp.nwg = int32_t((a->batch + rows - 1) / rows * ((kp.dtiles + wpg - 1) / wpg));
  if (a->disc == SSM_DISC_ZOH)
    hipLaunchKernelGGL((ssmk::k_step<N, InT, OutT, ssmk::kZoh>), dim3(kp.nwg),
                       dim3(ssmk::kWave * wpg), 0, s, kp);
  else
    hipLaunchKernelGGL((ssmk::k_step<N, InT, OutT, ssmk::kDeltaB>), dim3(kp.nwg),
                       dim3(ssmk::kWave * wpg), 0, s, kp);
  return launch_status("k_step");
}

template <int N>
ssm_status_t run_step_n(const ssm_step_args_t* a, const ssmk::StepParams& kp, hipStream_t s) {
  using ssmk::bf16_t;
  if (a->in_dtype == SSM_F32)
    return a->out_dtype == SSM_F32 ? run_step_t<N, float, float>(a, kp, s)
                                   : run_step_t<N, float, bf16_t>(a, kp, s);
  return a->out_dtype == SSM_F32 ? run_step_t<N, bf16_t, float>(a, kp, s)
                                 : run_step_t<N, bf16_t, bf16_t>(a, kp, s);
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

struct BwdPlan {
  int64_t Cf = 0;       // 16-step chunks (forward states recomputed from)
  int64_t Ts = 0;       // super-chunk length
  int64_t Cs = 0;       // super-chunks
  int64_t dtiles = 0;
  Grouping grp;         // of the 16-step forward carry walk
  Grouping rgrp;        // of the reverse carry walk over the super-chunks
  size_t off_hcar = 0, off_dsumf = 0, off_gsum = 0, off_dsums = 0, off_dAp = 0, off_dDp = 0,
         off_dBp = 0, off_dCp = 0, off_gS = 0, off_gB = 0, off_rgS = 0, off_rgB = 0, total = 0;
};

int ng_of(int64_t N) { return N < 4 ? 1 : int(N / 4); }

// Sizes assumed validated.
BwdPlan make_bwd_plan(int64_t Bt, int64_t L, int64_t D, int64_t N, int32_t super_chunk,
                      bool saved) {
  BwdPlan pl;
  const int64_t F = ssmk::kBwdFine;
  pl.dtiles = (D + ssmk::kWave - 1) / ssmk::kWave;
  if (L == 0 || Bt * D == 0) return pl;
  pl.Cf = (L + F - 1) / F;
  int64_t fines;   // fine chunks per super-chunk
  if (super_chunk > 0) {
    fines = super_chunk / F;
  } else {
    // the reverse summary runs one wave per (batch row, tile, super-chunk):
    // enough super-chunks to give it about kTargetWaves waves (the main pass,
    // with N / 4 waves each, then has more)
    const int64_t waves = Bt * pl.dtiles;
    const int64_t cs = std::max<int64_t>(1, std::min<int64_t>(kTargetWaves / waves, pl.Cf));
    fines = (pl.Cf + cs - 1) / cs;
    // Super-chunks longer than kBwdShortChunk steps are cut to that length
    // when the reverse carry walk then still crosses at most kGroupWalk of
    // them.  Measured (backward from kept states): 4 x 8192 x 2560 x 16 bf16
    // ZOH, 336-step super-chunks 2.35-2.41 ms, 128-step 2.23 ms; 8 x 2048 x
    // 1536 x 16 fp32 keeps its 112 steps (96-128 equal).  With many
    // super-chunks the sequential walk grows long: 1 x 2^20 x 512 x 16 keeps
    // 2048 steps (64-step super-chunks took 17.3 vs 10.0 ms).
    if (fines * F > kBwdShortChunk && (L + kBwdShortChunk - 1) / kBwdShortChunk <= kGroupWalk)
      fines = kBwdShortChunk / F;
    // With few chains the reverse walk is grouped (three short passes
    // instead of one chain per (b, d, n) across every super-chunk), and
    // super-chunks longer than kBwdLongChunk steps are cut to that length:
    // the main and reverse summary passes then get more, shorter waves.
    // Measured on 1 x 2^20 x 512 x 16 bf16 (backward from kept states).
    else if (fines * F > kBwdLongChunk && Bt * D * N < kGroupChains)
      fines = kBwdLongChunk / F;
  }
  // the reverse summary addresses a super-chunk's rows with 32-bit offsets
  const int64_t max_fines = std::max<int64_t>(1, kMaxChunkBytes / (D * 4) / F);
  fines = std::max<int64_t>(1, std::min(fines, max_fines));
  pl.Ts = fines * F;
  pl.Cs = (L + pl.Ts - 1) / pl.Ts;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t bt = size_t(Bt), d = size_t(D), n = size_t(N);
  // the forward states every 16 steps and their pass's buffers (none when
  // the caller hands in the forward scan's kept states)
  const size_t nf = saved ? 0 : size_t(pl.Cf - 1);
  pl.off_hcar = take(bt * nf * d * n * 4);
  pl.off_dsumf = take(bt * nf * d * 4);
  pl.off_gsum = take(bt * size_t(pl.Cs - 1) * d * n * 4);
  pl.off_dsums = take(bt * size_t(pl.Cs - 1) * d * 4);
  pl.off_dAp = take(bt * size_t(pl.Cs) * d * n * 4);
  pl.off_dDp = take(bt * size_t(pl.Cs) * d * 4);
  pl.off_dBp = take(bt * size_t(L) * size_t(pl.dtiles) * n * 4);
  pl.off_dCp = take(bt * size_t(L) * size_t(pl.dtiles) * n * 4);
  if (!saved) pl.grp = grouping(pl.Cf - 1, Bt * D * N);
  pl.off_gS = take(bt * size_t(pl.grp.G) * d * 4);
  pl.off_gB = take(bt * size_t(pl.grp.G) * d * n * 4);
  pl.rgrp = grouping(pl.Cs - 1, Bt * D * N);
  pl.off_rgS = take(bt * size_t(pl.rgrp.G) * d * 4);
  pl.off_rgB = take(bt * size_t(pl.rgrp.G) * d * n * 4);
  pl.total = off;
  return pl;
}

ssm_status_t check_bwd(const ssm_scan_bwd_args_t* a, BwdPlan* plan) {
  if (!a) return fail(SSM_ERR_NULL, "args is NULL");
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 0)
    return fail(SSM_ERR_SHAPE, "negative size: batch=%lld seqlen=%lld dim=%lld",
                (long long)a->batch, (long long)a->seqlen, (long long)a->dim);
  if (a->dstate < 1) return fail(SSM_ERR_SHAPE, "dstate must be >= 1 (got %lld)", (long long)a->dstate);
  if (a->in_dtype != SSM_F32 && a->in_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "unknown in_dtype %d", a->in_dtype);
  if (a->disc != SSM_DISC_DELTA_B && a->disc != SSM_DISC_ZOH)
    return fail(SSM_ERR_DTYPE, "unknown discretization %d", a->disc);
  if (!supported_n(a->dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate %lld not in {1,2,4,8,16}", (long long)a->dstate);
  if (a->reserved != 0) return fail(SSM_ERR_UNSUPPORTED, "reserved field must be 0");
  if (a->super_chunk < 0 || a->super_chunk % ssmk::kBwdFine != 0)
    return fail(SSM_ERR_UNSUPPORTED, "super_chunk must be a non-negative multiple of %d",
                ssmk::kBwdFine);
  int64_t bl, bld, bln, dn, bdn, blt;
  const int64_t dtiles = (a->dim + ssmk::kWave - 1) / ssmk::kWave;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) ||
      !mul_ok(bl, a->dstate, &bln) || !mul_ok(a->dim, a->dstate, &dn) ||
      !mul_ok(a->batch, dn, &bdn) || !mul_ok(bln, dtiles, &blt) || bld > INT64_MAX / 8 ||
      blt > INT64_MAX / 8 || bdn > INT64_MAX / 8)
    return fail(SSM_ERR_SHAPE, "sizes overflow");
  *plan = make_bwd_plan(a->batch, a->seqlen, a->dim, a->dstate, a->super_chunk,
                        a->h_saved != nullptr);
  if (!a->A || !a->dA) return fail(SSM_ERR_NULL, "A and dA are required");
  const bool work = a->seqlen > 0 && a->batch * a->dim > 0;
  if (work && (!a->x || !a->delta || !a->Bm || !a->Cm || !a->dy || !a->dx || !a->ddelta ||
               !a->dB || !a->dC))
    return fail(SSM_ERR_NULL, "x, delta, Bm, Cm, dy, dx, ddelta, dB and dC are required");
  const size_t in_sz = dtype_size(a->in_dtype);
  if (misaligned(a->x, in_sz) || misaligned(a->delta, in_sz) || misaligned(a->dy, in_sz) ||
      misaligned(a->Bm, 4) || misaligned(a->Cm, 4) || misaligned(a->A, 4) ||
      misaligned(a->Dskip, 4) || misaligned(a->h0, 4) || misaligned(a->dh_last, 4) ||
      misaligned(a->dx, 4) || misaligned(a->ddelta, 4) || misaligned(a->dA, 4) ||
      misaligned(a->dB, 4) || misaligned(a->dC, 4) || misaligned(a->dD, 4) ||
      misaligned(a->dh0, 4) || misaligned(a->workspace, 256) || misaligned(a->h_saved, 4))
    return fail(SSM_ERR_UNSUPPORTED,
                "misaligned pointer (element alignment; B, C 4 bytes; workspace 256 bytes)");
  const Range ins[] = {
      {a->x, size_t(bld) * in_sz},   {a->delta, size_t(bld) * in_sz}, {a->A, size_t(dn) * 4},
      {a->Bm, size_t(bln) * in_sz},  {a->Cm, size_t(bln) * in_sz},    {a->Dskip, size_t(a->dim) * 4},
      {a->h0, size_t(bdn) * 4},      {a->dy, size_t(bld) * in_sz},    {a->dh_last, size_t(bdn) * 4},
      {a->h_saved, size_t(bdn) * size_t(saved_count(a->seqlen)) * 4},
  };
  const Range outs[] = {
      {a->dx, size_t(bld) * 4}, {a->ddelta, size_t(bld) * 4}, {a->dA, size_t(dn) * 4},
      {a->dB, size_t(bln) * 4}, {a->dC, size_t(bln) * 4},     {a->dD, size_t(a->dim) * 4},
      {a->dh0, size_t(bdn) * 4},
  };
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(SSM_ERR_ALIAS, "a gradient overlaps an input");
    for (size_t k = i + 1; k < sizeof(outs) / sizeof(outs[0]); ++k)
      if (overlap(outs[i], outs[k])) return fail(SSM_ERR_ALIAS, "two gradients overlap");
  }
  if (!work) return SSM_OK;
  if (!a->workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", plan->total);
  if (a->workspace_bytes < plan->total)
    return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", a->workspace_bytes,
                plan->total);
  const Range ws{a->workspace, plan->total};
  for (const Range& r : ins)
    if (overlap(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps an input");
  for (const Range& r : outs)
    if (overlap(ws, r)) return fail(SSM_ERR_ALIAS, "workspace overlaps an output");
  const int64_t ng = ng_of(a->dstate);
  if (a->batch * plan->Cf * plan->dtiles > kMaxGrid ||
      a->batch * plan->Cs * plan->dtiles * ng > kMaxGrid || (bln + 255) / 256 > kMaxGrid ||
      (bdn * std::max<int64_t>(1, plan->grp.G) + 63) / 64 > kMaxGrid ||
      (bdn * std::max<int64_t>(1, plan->rgrp.G) + 63) / 64 > kMaxGrid)
    return fail(SSM_ERR_SHAPE, "problem too large for one launch");
  return SSM_OK;
}

template <int N, typename InT, int DISC>
ssm_status_t run_bwd(const ssm_scan_bwd_args_t* a, const BwdPlan& pl, hipStream_t s) {
  using namespace ssmk;
  char* ws = static_cast<char*>(a->workspace);
  const float thr = exact_threshold(a->disc, a->in_dtype);
  // forward states entering every 16-step chunk: kept by the forward scan,
  // or from the forward summary and carry passes run at that chunk length
  const bool saved = a->h_saved != nullptr;
  if (pl.Cf > 1 && !saved) {
    ScanParams fp{};
    fp.x = a->x;
    fp.delta = a->delta;
    fp.A = a->A;
    fp.Bm = a->Bm;
    fp.Cm = a->Cm;
    fp.h0 = a->h0;
    fp.dsum = reinterpret_cast<float*>(ws + pl.off_dsumf);
    fp.hsum = reinterpret_cast<float*>(ws + pl.off_hcar);
    fp.Bt = a->batch;
    fp.L = a->seqlen;
    fp.D = a->dim;
    fp.T = kBwdFine;
    fp.C = pl.Cf;
    fp.dtiles = int32_t(pl.dtiles);
    fp.exact_thr = thr;
    fp.dt_mode = kDtRaw;
    fp.nwg = int32_t(a->batch * (pl.Cf - 1) * pl.dtiles);
    hipLaunchKernelGGL((k_chunk_summary<N, InT, DISC, false>), dim3(fp.nwg), dim3(kWave), 0, s, fp);
    if (ssm_status_t st = launch_status("k_chunk_summary (backward)")) return st;
    fp.gS = reinterpret_cast<float*>(ws + pl.off_gS);
    fp.gB = reinterpret_cast<float*>(ws + pl.off_gB);
    if (ssm_status_t st = launch_combine<N>(fp, pl.grp, s)) return st;
  }
  BwdParams bp{};
  bp.x = a->x;
  bp.delta = a->delta;
  bp.A = a->A;
  bp.Bm = a->Bm;
  bp.Cm = a->Cm;
  bp.Dskip = a->Dskip;
  bp.h0 = a->h0;
  bp.dy = a->dy;
  bp.dh_last = a->dh_last;
  bp.dx = a->dx;
  bp.ddelta = a->ddelta;
  bp.dA = a->dA;
  bp.dB = a->dB;
  bp.dC = a->dC;
  bp.dD = a->dD;
  bp.dh0 = a->dh0;
  bp.hcar = saved ? a->h_saved : reinterpret_cast<const float*>(ws + pl.off_hcar);
  bp.gsum = reinterpret_cast<float*>(ws + pl.off_gsum);
  bp.dsum_s = reinterpret_cast<float*>(ws + pl.off_dsums);
  bp.dAp = reinterpret_cast<float*>(ws + pl.off_dAp);
  bp.dDp = reinterpret_cast<float*>(ws + pl.off_dDp);
  bp.dBp = reinterpret_cast<float*>(ws + pl.off_dBp);
  bp.dCp = reinterpret_cast<float*>(ws + pl.off_dCp);
  bp.rgS = reinterpret_cast<float*>(ws + pl.off_rgS);
  bp.rgB = reinterpret_cast<float*>(ws + pl.off_rgB);
  bp.rG = pl.rgrp.G;
  bp.rgsz = pl.rgrp.gsz;
  bp.Bt = a->batch;
  bp.L = a->seqlen;
  bp.D = a->dim;
  bp.Ts = pl.Ts;
  bp.Cs = pl.Cs;
  bp.Cf = pl.Cf;
  bp.dtiles = int32_t(pl.dtiles);
  bp.exact_thr = thr;
  if (pl.Cs > 1) {
    bp.nwg = int32_t(a->batch * (pl.Cs - 1) * pl.dtiles);
    hipLaunchKernelGGL((k_bwd_summary<N, InT, DISC>), dim3(bp.nwg), dim3(kWave), 0, s, bp);
    if (ssm_status_t st = launch_status("k_bwd_summary")) return st;
    const int64_t chains = a->batch * a->dim * N;
    if (pl.rgrp.G > 0) {
      const int64_t gchains = chains * pl.rgrp.G;
      hipLaunchKernelGGL((k_bwd_rgroups<N>), dim3(uint32_t((gchains + 63) / 64)), dim3(kWave), 0,
                         s, bp);
      if (ssm_status_t st = launch_status("k_bwd_rgroups")) return st;
      hipLaunchKernelGGL((k_bwd_rtop<N>), dim3(uint32_t((chains + 63) / 64)), dim3(kWave), 0, s,
                         bp);
      if (ssm_status_t st = launch_status("k_bwd_rtop")) return st;
      hipLaunchKernelGGL((k_bwd_rapply<N>), dim3(uint32_t((gchains + 63) / 64)), dim3(kWave), 0,
                         s, bp);
      if (ssm_status_t st = launch_status("k_bwd_rapply")) return st;
    } else {
      hipLaunchKernelGGL((k_bwd_combine<N>), dim3(uint32_t((chains + 63) / 64)), dim3(kWave), 0,
                         s, bp);
      if (ssm_status_t st = launch_status("k_bwd_combine")) return st;
    }
  }
  constexpr int NG = BwdLayout<N>::NG;
  bp.nwg = int32_t(a->batch * pl.Cs * pl.dtiles);
  hipEvent_t e0 = static_cast<hipEvent_t>(a->ev_main_start);
  hipEvent_t e1 = static_cast<hipEvent_t>(a->ev_main_stop);
  if (e0 && hipEventRecord(e0, s) != hipSuccess) return fail(SSM_ERR_HIP, "hipEventRecord failed");
  hipLaunchKernelGGL((k_bwd_main<N, InT, DISC>), dim3(bp.nwg), dim3(kWave * NG), 0, s, bp);
  if (ssm_status_t st = launch_status("k_bwd_main")) return st;
  if (e1 && hipEventRecord(e1, s) != hipSuccess) return fail(SSM_ERR_HIP, "hipEventRecord failed");
  const int64_t nbc = a->batch * a->seqlen * N;
  hipLaunchKernelGGL((k_bwd_reduce_bc<N>), dim3(uint32_t((nbc + 255) / 256)), dim3(256), 0, s, bp);
  if (ssm_status_t st = launch_status("k_bwd_reduce_bc")) return st;
  const int64_t nad = a->dim * N + a->dim;
  hipLaunchKernelGGL((k_bwd_reduce_ad<N>), dim3(uint32_t((nad + kWave - 1) / kWave)),
                     dim3(kWave * kRedWaves), 0, s, bp);
  return launch_status("k_bwd_reduce_ad");
}

template <int N>
ssm_status_t run_bwd_n(const ssm_scan_bwd_args_t* a, const BwdPlan& pl, hipStream_t s) {
  using ssmk::bf16_t;
  if (a->in_dtype == SSM_F32)
    return a->disc == SSM_DISC_ZOH ? run_bwd<N, float, ssmk::kZoh>(a, pl, s)
                                   : run_bwd<N, float, ssmk::kDeltaB>(a, pl, s);
  return a->disc == SSM_DISC_ZOH ? run_bwd<N, bf16_t, ssmk::kZoh>(a, pl, s)
                                 : run_bwd<N, bf16_t, ssmk::kDeltaB>(a, pl, s);
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

size_t ssm_scan_workspace_size(const ssm_scan_args_t* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->dim < 0 || a->dstate < 1 || a->chunk_len < 0)
    return 0;
  int64_t bl, bld, bdn;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) ||
      !mul_ok(a->batch, a->dim * a->dstate, &bdn))
    return 0;
  return one_pass_plan(a, make_plan(a->batch, a->seqlen, a->dim, a->dstate, a->chunk_len)).ws_total;
}

int64_t ssm_scan_plan_chunk_len(const ssm_scan_args_t* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->dim < 0 || a->dstate < 1 || a->chunk_len < 0)
    return 0;
  int64_t bl, bld;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld)) return 0;
  return one_pass_plan(a, make_plan(a->batch, a->seqlen, a->dim, a->dstate, a->chunk_len)).T;
}

int32_t ssm_scan_plan_lane_scan(const ssm_scan_args_t* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->dim < 0 || a->dstate < 1 || a->chunk_len < 0)
    return 0;
  int64_t bl, bld;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld)) return 0;
  return one_pass_plan(a, make_plan(a->batch, a->seqlen, a->dim, a->dstate, a->chunk_len)).wave ? 1 : 0;
}

}  // extern "C"

namespace {

// The forward scan of checked arguments with plan `pl`, its chunk summaries
// in `ws` (pl.ws_total bytes; unused when the plan has one chunk).
ssm_status_t scan_fwd_run(const ssm_scan_args_t* a, const Plan& pl, void* ws, hipStream_t s) {
  const int64_t BD = a->batch * a->dim;
  if (BD == 0) return SSM_OK;
  if (a->seqlen == 0) {
    if (a->h_last) {
      const int64_t n = BD * a->dstate;
      hipLaunchKernelGGL(ssmk::k_state_copy, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s,
                         a->h_last, a->h0, n);
      if (ssm_status_t st = launch_status("k_state_copy")) return st;
    }
    if (a->conv_w && a->conv_state_out && a->conv_k > 1) {
      const int64_t n = BD * (a->conv_k - 1);
      hipLaunchKernelGGL(ssmk::k_state_copy, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s,
                         a->conv_state_out, a->conv_state_in, n);
      if (ssm_status_t st = launch_status("k_state_copy")) return st;
    }
    return SSM_OK;
  }
  ssmk::ScanParams kp{};
  kp.x = a->x;
  kp.delta = a->delta;
  kp.A = a->A;
  kp.Bm = a->Bm;
  kp.Cm = a->Cm;
  kp.Dskip = a->Dskip;
  kp.h0 = a->h0;
  kp.h_last = a->h_last;
  kp.y = a->y;
  kp.conv_w = a->conv_w;
  kp.conv_b = a->conv_w ? a->conv_b : nullptr;
  kp.conv_k = a->conv_w ? a->conv_k : 0;
  kp.dsum = pl.C > 1 ? static_cast<float*>(ws) : nullptr;
  kp.hsum = pl.C > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + pl.ws_dsum) : nullptr;
  if (pl.grp.G > 0) {
    char* wsb = static_cast<char*>(ws);
    kp.gS = reinterpret_cast<float*>(wsb + pl.ws_dsum + pl.ws_hsum);
    kp.gB = reinterpret_cast<float*>(wsb + pl.ws_dsum + pl.ws_hsum + pl.ws_gS);
  }
  kp.Bt = a->batch;
  kp.L = a->seqlen;
  kp.D = a->dim;
  kp.T = pl.T;
  kp.C = pl.C;
  kp.dtiles = int32_t(pl.dtiles);
  kp.exact_thr = exact_threshold(a->disc, a->in_dtype);
  kp.dt_bias = a->delta_bias;
  kp.dt_mode = dt_mode_of(a->delta_bias, a->delta_softplus);
  kp.z = a->z;
  kp.cs_in = a->conv_w ? a->conv_state_in : nullptr;
  kp.cs_out = a->conv_w ? a->conv_state_out : nullptr;
  kp.nsave = saved_count(a->seqlen);
  kp.hsave = kp.nsave > 0 ? a->h_saved : nullptr;
  switch (a->dstate) {
    case 1: return dispatch_types<1>(a, kp, pl, s);
    case 2: return dispatch_types<2>(a, kp, pl, s);
    case 4: return dispatch_types<4>(a, kp, pl, s);
    case 8: return dispatch_types<8>(a, kp, pl, s);
    default: return dispatch_types<16>(a, kp, pl, s);
  }
}

}  // namespace

extern "C" {

ssm_status_t ssm_scan_fwd(const ssm_scan_args_t* a, void* hip_stream) {
  g_msg[0] = '\0';
  Plan pl;
  if (ssm_status_t st = check_scan(a, &pl)) return st;
  return scan_fwd_run(a, pl, a->workspace, static_cast<hipStream_t>(hip_stream));
}

ssm_status_t ssm_scan_fwd_noalloc(const ssm_scan_args_t* a, void* hip_stream) {
  g_msg[0] = '\0';
  Plan pl;
  if (ssm_status_t st = check_scan(a, &pl, true)) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  void* ws = nullptr;
  if (pl.ws_total > 0 && a->seqlen > 0 && a->batch * a->dim > 0) {
    if (ssm_status_t st = scratch_address(s, &ws)) return st;
  }
  return scan_fwd_run(a, pl, ws, s);
}

ssm_status_t ssm_step(const ssm_step_args_t* a, void* hip_stream) {
  g_msg[0] = '\0';
  if (ssm_status_t st = check_step(a)) return st;
  if (a->batch * a->dim == 0) return SSM_OK;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  ssmk::StepParams kp{};
  kp.x = a->x;
  kp.delta = a->delta;
  kp.A = a->A;
  kp.Bm = a->Bm;
  kp.Cm = a->Cm;
  kp.Dskip = a->Dskip;
  kp.h = a->h;
  kp.y = a->y;
  kp.Bt = a->batch;
  kp.D = a->dim;
  kp.exact_thr = exact_threshold(a->disc, a->in_dtype);
  kp.dt_bias = a->delta_bias;
  kp.dt_mode = dt_mode_of(a->delta_bias, a->delta_softplus);
  kp.z = a->z;
  kp.conv_k = a->conv_w ? a->conv_k : 0;
  kp.conv_w = a->conv_w;
  kp.conv_b = a->conv_w ? a->conv_b : nullptr;
  kp.conv_state = a->conv_w ? a->conv_state : nullptr;
  switch (a->dstate) {
    case 1: return run_step_n<1>(a, kp, s);
    case 2: return run_step_n<2>(a, kp, s);
    case 4: return run_step_n<4>(a, kp, s);
    case 8: return run_step_n<8>(a, kp, s);
    default: return run_step_n<16>(a, kp, s);
  }
}

size_t ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args_t* a) {
  if (!a || a->batch < 0 || a->seqlen < 0 || a->dim < 0 || a->dstate < 1 ||
      a->super_chunk < 0 || a->super_chunk % ssmk::kBwdFine != 0)
    return 0;
  int64_t bl, bld, bln;
  if (!mul_ok(a->batch, a->seqlen, &bl) || !mul_ok(bl, a->dim, &bld) ||
      !mul_ok(bl, a->dstate, &bln) || bln > INT64_MAX / 64)
    return 0;
  return make_bwd_plan(a->batch, a->seqlen, a->dim, a->dstate, a->super_chunk,
                       a->h_saved != nullptr)
      .total;
}

ssm_status_t ssm_scan_bwd(const ssm_scan_bwd_args_t* a, void* hip_stream) {
  g_msg[0] = '\0';
  BwdPlan pl;
  if (ssm_status_t st = check_bwd(a, &pl)) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t DN = a->dim * a->dstate;
  if (a->seqlen == 0 || a->batch * a->dim == 0) {
    // no token: dA, dD are zero and the gradient of h0 is dh_last
    if (DN > 0) {
      hipLaunchKernelGGL(ssmk::k_state_copy, dim3(uint32_t((DN + 255) / 256)), dim3(256), 0, s,
                         a->dA, nullptr, DN);
      if (ssm_status_t st = launch_status("k_state_copy")) return st;
    }
    if (a->dD && a->dim > 0) {
      hipLaunchKernelGGL(ssmk::k_state_copy, dim3(uint32_t((a->dim + 255) / 256)), dim3(256), 0,
                         s, a->dD, nullptr, a->dim);
      if (ssm_status_t st = launch_status("k_state_copy")) return st;
    }
    const int64_t n = a->batch * DN;
    if (a->dh0 && n > 0) {
      hipLaunchKernelGGL(ssmk::k_state_copy, dim3(uint32_t((n + 255) / 256)), dim3(256), 0, s,
                         a->dh0, a->dh_last, n);
      if (ssm_status_t st = launch_status("k_state_copy")) return st;
    }
    return SSM_OK;
  }
  switch (a->dstate) {
    case 1: return run_bwd_n<1>(a, pl, s);
    case 2: return run_bwd_n<2>(a, pl, s);
    case 4: return run_bwd_n<4>(a, pl, s);
    case 8: return run_bwd_n<8>(a, pl, s);
    default: return run_bwd_n<16>(a, pl, s);
  }
}

const char* ssm_status_string(ssm_status_t s) {
  // Any integer may arrive here; an enum object holding a value outside its
  // enumerators' range must not be read as the enum, so read its bits.
  static_assert(sizeof(s) == sizeof(int), "ssm_status_t is int-sized");
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid or overflowing sizes";
    case SSM_ERR_DTYPE: return "unknown dtype or discretization";
    case SSM_ERR_UNSUPPORTED: return "unsupported argument";
    case SSM_ERR_ALIAS: return "output overlaps another buffer";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ssm_last_error_message(void) { return g_msg; }

}  // extern "C"
