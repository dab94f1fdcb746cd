// Fused selective-scan forward for MI355X (gfx950, CDNA4) and its C ABI.
//
// The method (the pwwt.cn article, sections 1.1, 2.1-2.4 and 3.1; the
// bjdmk.com.cn article, sections 2.2-2.4): for each batch row b, channel d and
// state n the diagonal recurrence h_t = exp(delta_t*A[d,n]) h_{t-1} +
// delta_t B[b,t,n] x[b,t,d] is an affine map h -> a*h + b per step.  Affine
// maps compose associatively, (a1,b1) then (a2,b2) = (a1*a2, a2*b1 + b2), so
// the time axis can be cut into pieces that are folded independently and then
// joined by carrying the state from piece to piece.
//
// Work mapping (one workgroup = one batch row x 16 consecutive channels):
//  * A lane owns one channel and 16 states (dstate = 16*G; lane row r of the
//    wave picks the state group g = r % G) and K consecutive time steps (the
//    time sub-chunk q = r / G of the wave).  A tile of the time axis is
//    SUB = W*(4/G) sub-chunks of K steps.
//  * Pass 1 (per lane, serial over K steps): Abar = exp2(delta*A*log2e) for
//    each state, kept in registers; the sub-chunk's folded b_total and its
//    sum of delta go to LDS.  The G state-group rows of a sub-chunk split the
//    per-(step, channel) work -- loading x and delta, softplus, u = delta*x --
//    K/G steps each and exchange the results across rows.
//  * Carry walk: one lane per (channel, state) walks the SUB sub-chunks of the
//    tile in time order with the pair (a_prod, b_total), a_prod =
//    exp2(A*log2e*sum(delta)), leaving each sub-chunk's incoming state in LDS
//    and keeping the carry in a register from tile to tile (the serial
//    chunk-to-chunk carry of the chunked scan).
//  * Pass 2 (per lane, serial over K steps): h = Abar*h + delta*B*x from the
//    incoming state using the cached Abar (so each state update costs exactly
//    one exp), y = C.h + D*x.  At dstate 16 (serial walk) the sub-chunk's
//    last step, whose state nothing reads, splits its readout as
//    C.(Abar*h) + u*(C.B), with the dot product C.B summed across the row.
//  * B and C are shared by the 16 channels of a workgroup: lane s of each
//    16-lane row loads B[b,t,16g+s] and C[b,t,16g+s] for that row's step.  B's
//    per-state operand is taken with a DPP row broadcast (row_newbcast:s)
//    fused into the multiply; C is staged in LDS as fp32 after pass 1 and
//    read back as quads by pass 2's readout (plain FMAs, 5 % faster than the
//    DPP broadcast at every dstate).
//  * Padded steps (t >= valid_len) get delta = 0, u = 0 and B = 0, i.e. the
//    identity pair (1, 0) (pwwt.cn section 2.3, identity element instead of a
//    branch), and y = +0 there.  Tiles that lie wholly in the padding are not
//    loaded at all.
//  * With G > 1 the 16-state partial sums of y from the G state-group rows are
//    reduce-scattered with v_permlane16_swap / v_permlane32_swap in a fixed
//    order, so that each row holds the totals of the steps it stores.
//  * The carry walk can be replaced by a log-depth (Hillis-Steele) scan across
//    each wave's sub-chunks with a walk over the wave totals only
//    (extras.combine; slower on this GPU, kept as an option).
//  * Rows of different lengths at exactly two workgroups per CU are dealt so
//    that each CU holds one long and one short row (length_paired_row).
//  * Small batches with long sequences split the time axis over workgroups:
//    a fold kernel over the first parts, then every part from its incoming
//    state.
//
// All arithmetic is fp32; exp is v_exp_f32 (2^x) after a log2(e) prescale.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "ssm_internal.h"
#include "ssm_scan.h"

namespace {

struct FwdParams {
  const void* x;
  const void* delta;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const int32_t* valid_len;
  void* y;
  float* h_last;
  const float* h0;
  const float* delta_bias;
  const void* z;
  float* chunk_states;
  int64_t chunk_len;  // steps per chunk of chunk_states: a multiple of K dividing the tile
  // Time split across workgroups: the sequence is cut into n_parts parts of
  // part_len steps (a multiple of the tile; part_len = L when unsplit).  ws
  // holds, per part boundary, what the fold kernel leaves for the next parts.
  float* ws;
  int64_t part_len;
  int32_t n_parts;
  int64_t L;
  int32_t nb;
  int32_t nd;
  int32_t n_cg;  // channel groups of 16 per batch row
  int32_t softplus;
  int32_t clamp;
  float dmin;
  float dmax;
  int32_t wave_scan;  // the main kernel combines sub-chunks with the log-depth wave scan
  int32_t pair_rows;  // rows of different lengths: pair the longest with the shortest on each CU
};

// ---- the kernel ----------------------------------------------------------

// 128 VGPRs, so that two 8-wave workgroups share a CU (4 waves per SIMD).
// dstate 32 and 64 spill a few registers per tile to get there (measured: the
// second workgroup per CU is worth far more than the spills cost).
constexpr int kMinWavesPerSimd = 4;
// The fold kernel keeps no Abar cache (~80 VGPRs) and one record buffer, so
// three 8-wave workgroups share a CU.
constexpr int kFoldWavesPerSimd = 6;

// Sub-chunks per batch of the carry walk (2, or a multiple of 4): 8 at
// dstate 16 and 32, 2 at dstate 64, where every thread walks two (channel,
// state) pairs.  Measured (B8 L4096 D1024 forward, bf16, single record
// buffer; us at dstate 16 / 32 / 64): batches of 8 186.0 / 379.5 / 835.6, of 4
// 186.7 / 384.7 / 773.6, of 2 188.2 / 387.1 / 751.5; on the current sources
// at dstate 64, 712 / 706 / 695.
template <int G>
constexpr int kWalkBatch = G == 4 ? 2 : 8;

// FOLD: the fold kernel of the time split -- pass 1 and the carry walk only,
// over parts 0 .. n_parts-2, leaving each part's carry-out (part 0, from h0)
// or its b_total and delta sum (later parts, from zero) in the workspace.
// Otherwise the full forward over every part, each starting from the state
// the workspace gives for its first step.
// WSCAN: the cross-sub-chunk combine as a log-depth (Hillis-Steele) scan of
// the (a_prod, b_total) pairs across the sub-chunks of each wave, through
// v_permlane16/32_swap, with only the wave totals walked serially through LDS;
// otherwise the serial walk over every sub-chunk of the tile.
template <typename IO, int G, int K, int W, bool SOFTPLUS, bool CLAMP, bool GATE, bool FOLD, bool WSCAN = false>
__global__ __launch_bounds__(64 * W, FOLD ? kFoldWavesPerSimd : kMinWavesPerSimd) void ssm_fwd_kernel(FwdParams p) {
  constexpr int N = 16 * G;             // states per channel
  constexpr int QR = 4 / G;             // time sub-chunks per wave
  constexpr int SUB = W * QR;           // sub-chunks per tile
  constexpr int T = SUB * K;            // steps per tile
  constexpr int NS = N + 4;             // padded row stride of the A table in floats
  constexpr int SDS = SUB + 4;          // padded row stride of the sub-chunk delta sums
  static_assert(SUB % 4 == 0, "sub-chunk records are read as quads");
  constexpr int AGG = SUB * 16 * N;     // floats of one tile's sub-chunk records
  constexpr int PAIRS = 16 * N;         // (channel, state) pairs of the workgroup
  constexpr int NT = 64 * W;            // threads
  constexpr int PPL = (PAIRS + NT - 1) / NT;
  constexpr int E = Elem<IO>::kBytes;

  // Per tile and sub-chunk j, channel c, state n: b_total, then overwritten by
  // the walk with the incoming state.  Stored as float4 quads,
  // index ((j * N/4 + n/4) * 16 + c) * 4 + n%4, so that a row of 16 lanes
  // writes one quad each into 64 consecutive dwords, and a walk wave reading
  // 16 channels x 4 states touches 64 consecutive dwords (see pair_of).
  // One buffer: after
  // the walk, a lane reads only its own sub-chunk's slot, and it writes that
  // slot again only in the next tile's pass 1; every other access (the walk,
  // the sub-chunk delta sums) lies between the two barriers of a tile.  (Two
  // alternating buffers: the same time at dstate 16 and 32, 2 % slower at 64,
  // more registers spilled.)  The fold kernel, which has no pass 2, takes a
  // barrier after the walk instead.
  __shared__ __attribute__((aligned(16))) float agg_b[AGG];
  // WSCAN: each wave's incoming state, per tile, from the walk over the wave
  // totals (same quad layout as the records, one slot per wave).
  __shared__ __attribute__((aligned(16))) float wave_in[WSCAN && !FOLD ? W * 16 * N : 4];
  // Sum of delta over each sub-chunk, channel-major (row stride SDS) so that a
  // walk lane reads its channel's sub-chunks as consecutive quads.
  __shared__ __attribute__((aligned(16))) float agg_sd[16 * SDS];
  __shared__ __attribute__((aligned(16))) float a2s[16 * NS];  // A * log2(e) for the workgroup's channels
  __shared__ int32_t row_lens[64], row_order[64];  // length pairing of rows (at most 64 rows)
  // C of the tile as fp32, [step][state] with a padded row stride (the four
  // sub-chunks a wave's rows read fall on different banks): pass 2's readout
  // reads it as quads and uses plain FMAs instead of DPP row broadcasts.  A
  // wave reads only the steps of its own sub-chunks and rewrites them only in
  // its next tile's pass 1, so one buffer suffices.
  constexpr int CS = N + 4;
  __shared__ __attribute__((aligned(16))) float c_s[FOLD ? 4 : T * CS];

  // Workgroup -> (time part, batch row, channel group).  Workgroups are dealt
  // to the 8 XCDs round-robin; consecutive logical ids are kept on one XCD so
  // that neighbouring channel groups (which share 128-byte lines of x, delta
  // and y) share that XCD's L2.
  const int64_t groups = static_cast<int64_t>(p.nb) * p.n_cg;
  const int64_t total = groups * (FOLD ? p.n_parts - 1 : p.n_parts);
  const int64_t bid = blockIdx.x;
  const int64_t per_xcd = total / 8;
  const int64_t logical = (bid < per_xcd * 8) ? (bid % 8) * per_xcd + bid / 8 : bid;
  const int part = static_cast<int>(logical / groups);
  int b = static_cast<int>((logical % groups) / p.n_cg);
  int cg = static_cast<int>(logical % p.n_cg);
  // rows of different lengths: the longest row shares its CUs with the
  // shortest (309 -> 232 us on 16 rows of 128-8192 steps, 512 channels)
  if (!FOLD && p.pair_rows) length_paired_row(bid, groups, p.n_cg, p.nb, p.L, p.valid_len, row_lens, row_order, b, cg);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int r = lane >> 4;
  const int c = lane & 15;
  const int q = r / G;
  const int g = r % G;
  const int j = w * QR + q;  // sub-chunk index within the tile
  const int d = cg * 16 + c;
  const int nd = p.nd;
  // This workgroup's steps [t_begin, t_begin + L) of the sequence; below, every
  // step index is relative to t_begin.
  const int64_t t_begin = part * p.part_len;
  const int64_t L = (p.L - t_begin < p.part_len) ? p.L - t_begin : p.part_len;

  int64_t len = p.L;  // valid steps of the row, then of the part
  if (p.valid_len != nullptr) {
    const int64_t v = p.valid_len[b];
    len = v < 0 ? 0 : (v > p.L ? p.L : v);
  }
  len = len - t_begin;
  len = len < 0 ? 0 : (len > L ? L : len);

  for (int k = tid; k < 16 * N; k += NT) {
    const int cc = k / N, n = k % N;
    a2s[cc * NS + n] = -expf(p.A_log[static_cast<int64_t>(cg * 16 + cc) * N + n]) * kLog2e;
  }
  // D*x is added once per (t, d): by the first state-group row only.
  const float dskip = (p.D != nullptr && g == 0) ? p.D[d] : 0.0f;
  const float dbias = (p.delta_bias != nullptr) ? p.delta_bias[d] : 0.0f;

  // The walk lane's (channel, state) pair k: each group of 64 pairs is 16
  // channels x 4 states, state fastest, so that a wave's lanes touch 64
  // consecutive words of a record slot (the LDS serves a 32-lane half per
  // cycle from 32 banks: with the channel fastest, channels c and c + 8 shared
  // a bank, 67 conflict cycles per wave and tile at dstate 16; this way 2, and
  // 1-2 % faster at every dstate).
  auto pair_of = [&](int k, int& cc, int& n) {
    const int pr = tid + k * NT;
    cc = (pr & 63) >> 2;
    n = 4 * (pr >> 6) + (pr & 3);
  };
  auto pair_valid = [&](int k) { return PAIRS % NT == 0 || tid + k * NT < PAIRS; };
  // Offset of pair k within the workgroup's 16 x N block of a [.., dim, dstate]
  // tensor (the block itself starts at a wave-uniform address).
  auto pair_offset = [&](int k) {
    int cc, n;
    pair_of(k, cc, n);
    return static_cast<uint32_t>(cc * N + n);
  };
  const int64_t state_block = (static_cast<int64_t>(b) * nd + cg * 16) * N;
  // Workspace: n_parts - 1 state blocks [nb, nd, N] -- block 0 is the state
  // entering part 1, block q >= 1 the b_total of part q folded from zero --
  // then the delta sums of parts 1 .. n_parts-2, [n_parts - 2, nb, nd].
  const int64_t ws_block = static_cast<int64_t>(p.nb) * nd * N;
  float* const ws_sd = p.ws + (p.n_parts - 1) * ws_block;

  float carry[PPL];
#pragma unroll
  for (int k = 0; k < PPL; ++k) carry[k] = 0.0f;
  if (part == 0) {
    if (p.h0 != nullptr) {
      const float* h0b = p.h0 + state_block;
#pragma unroll
      for (int k = 0; k < PPL; ++k)
        if (pair_valid(k)) carry[k] = h0b[pair_offset(k)];
    }
  } else if (!FOLD) {
    // The state entering this part: the carry into part 1, then the parts in
    // between composed as affine maps (a_prod = exp2(A log2(e) sum(delta)),
    // b_total), in time order -- the chunk-to-chunk carry of the chunked scan.
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      if (pair_valid(k)) {
        int cc, n;
        pair_of(k, cc, n);
        const float a2 = -expf(p.A_log[static_cast<int64_t>(cg * 16 + cc) * N + n]) * kLog2e;
        float cr = p.ws[state_block + pair_offset(k)];
        for (int qp = 1; qp < part; ++qp) {
          const float sdq = ws_sd[(static_cast<int64_t>(qp - 1) * p.nb + b) * nd + cg * 16 + cc];
          cr = __builtin_fmaf(fast_exp2(a2 * sdq), cr, p.ws[qp * ws_block + state_block + pair_offset(k)]);
        }
        carry[k] = cr;
      }
    }
  }
  float part_sd[PPL];  // FOLD, part >= 1: the part's delta sum for the pair's channel
#pragma unroll
  for (int k = 0; k < PPL; ++k) part_sd[k] = 0.0f;
  // Chunk-boundary states: the state after the last step of every chunk of
  // chunk_len steps (chunks are numbered from the start of the sequence; a
  // chunk boundary is always a sub-chunk boundary, and a part starts on a tile
  // boundary).  The last chunk may end past L: past the valid length the state
  // no longer changes.
  const int64_t n_chunks = (p.L + p.chunk_len - 1) / p.chunk_len;
  const bool want_chunks = !FOLD && p.chunk_states != nullptr;
  const int clj = static_cast<int>(p.chunk_len / K);  // sub-chunks per chunk (divides SUB)
  // Stores pair k's state as that of chunk ci (ignored past the last chunk).
  auto store_chunk = [&](int64_t ci, int k, float v) {
    if (ci < n_chunks)
      p.chunk_states[((static_cast<int64_t>(b) * n_chunks + ci) * nd + cg * 16) * N + pair_offset(k)] = v;
  };

  // Buffer resources of this batch row's x, delta, y, B and C, and the lane's
  // byte offsets of its first step in a tile.
  const int64_t xd_step = static_cast<int64_t>(nd) * E;  // bytes between consecutive steps of x/delta/y
  const int64_t bc_step = static_cast<int64_t>(N) * E;   // ... of B/C
  // The part's rows start at b * (whole row) + t_begin * step and span L steps.
  const int64_t xd_base = (b * p.L + t_begin) * xd_step, bc_base = (b * p.L + t_begin) * bc_step;
  const int64_t xd_row = L * xd_step, bc_row = L * bc_step;
  const rsrc_t rx = make_rsrc(static_cast<const char*>(p.x) + xd_base, xd_row);
  const rsrc_t rd = make_rsrc(static_cast<const char*>(p.delta) + xd_base, xd_row);
  const rsrc_t ry = make_rsrc(FOLD ? nullptr : static_cast<char*>(p.y) + xd_base, FOLD ? 0 : xd_row);
  const rsrc_t rb = make_rsrc(static_cast<const char*>(p.B) + bc_base, bc_row);
  const rsrc_t rc = make_rsrc(FOLD ? nullptr : static_cast<const char*>(p.C) + bc_base, FOLD ? 0 : bc_row);
  const rsrc_t rz = make_rsrc(GATE && !FOLD ? static_cast<const char*>(p.z) + xd_base : nullptr,
                              GATE && !FOLD ? xd_row : 0);
  const uint32_t off_xd = static_cast<uint32_t>((j * K * nd + d) * E);
  const uint32_t off_bc = static_cast<uint32_t>((j * K * N + 16 * g + c) * E);

  // x and delta are loaded and discretised once per (step, channel): the G
  // state-group rows of a sub-chunk share its steps, so row g takes steps
  // g*KG .. g*KG + KG-1 and the rows exchange the results (share_rows).
  constexpr int KG = K / G;
  static_assert(KG * G == K, "each state-group row discretises K / G steps");
  const uint32_t off_xd_own = off_xd + static_cast<uint32_t>(g * KG * nd * E);
  // x and delta of the lane's own KG steps in the tile starting at t_tile, as
  // the loaded bits (widened to fp32 where they are used, so that a prefetch
  // does not wait for its data on the spot).  Steps at or beyond len read as 0
  // (never loaded).
  auto load_raw = [](rsrc_t r, uint32_t voff, uint32_t soff) -> uint32_t {
    if constexpr (E == 2)
      return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kCached);
    else
      return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kCached);
  };
  auto widen = [](uint32_t u) -> float { return __builtin_bit_cast(float, E == 2 ? u << 16 : u); };
  auto load_xd = [&]<bool FULL>(int64_t t_tile, uint32_t (&xr)[KG], uint32_t (&dr)[KG]) {
    const int64_t left = len - t_tile - j * K;
#pragma unroll
    for (int m = 0; m < KG; ++m) {
      const bool ok = FULL || g * KG + m < left;
      const uint32_t sx = static_cast<uint32_t>((t_tile + m) * xd_step);
      xr[m] = ok ? load_raw(rx, off_xd_own, sx) : 0u;
      dr[m] = ok ? load_raw(rd, off_xd_own, sx) : 0u;
    }
  };
  // The values of all K steps of the sub-chunk from the rows that computed
  // them (own: this lane's KG steps): at G = 2 the row pair exchanges through
  // v_permlane16_swap; at G = 4 each of the four rows' steps are gathered with
  // one v_permlane16_swap and two v_permlane32_swap.
  auto share_rows = [](const float (&own)[KG], float (&all)[K]) __attribute__((always_inline)) {
    if constexpr (G == 1) {
#pragma unroll
      for (int i = 0; i < K; ++i) all[i] = own[i];
    } else if constexpr (G == 2) {
#pragma unroll
      for (int m = 0; m < KG; ++m) rows_swap16(own[m], all[m], all[KG + m]);  // rows 2q and 2q+1
    } else {
#pragma unroll
      for (int m = 0; m < KG; ++m) {
        float lo, hi;
        rows_swap16(own[m], lo, hi);  // rows [0, 0, 2, 2] and [1, 1, 3, 3]
        rows_swap32(lo, all[m], all[2 * KG + m]);
        rows_swap32(hi, all[KG + m], all[3 * KG + m]);
      }
    }
  };

  // Log-depth combine across the wave's QR sub-chunks (WSCAN).  Each lane
  // holds its sub-chunk's b_total (bt, folded from zero), its delta sum (sd)
  // and the Abar of its K steps (ab); a_prod is their product.  An inclusive
  // Hillis-Steele scan over the sub-chunks (rows q*G + g of the wave) combines
  // each with the one 1, then 2 sub-chunks earlier -- b updated before a --
  // taking the partner's values from v_permlane16_swap and v_permlane32_swap
  // (a sub-chunk is 16 lanes at dstate 16, 32 at dstate 32); the delta sums
  // are scanned alongside.  Each lane parks its
  // inclusive b in its record slot (the last sub-chunk's is the wave total),
  // the wave totals are walked serially in time order (W of them per tile,
  // the carry kept across tiles) leaving each wave's incoming state in
  // wave_in, and each lane then forms the state after its sub-chunk, with the
  // inclusive a_prod recomputed as exp2(A log2(e) * inclusive delta sum); its
  // own incoming state is the one after the sub-chunk before it.
  // WSCAN: a lane's wave incoming state, its parked inclusive b and A*log2(e)
  // for states s .. s+3 (valid from the walk until the next tile's pass 1)
  auto ws_after_own = [&](int s, float4& hw4, float4& bi4, float4& a24) __attribute__((always_inline)) {
    hw4 = *reinterpret_cast<const float4*>(wave_in + ((w * (N / 4) + 4 * g) * 16 + c) * 4 + s * 16);
    bi4 = *reinterpret_cast<const float4*>(agg_b + ((j * (N / 4) + 4 * g) * 16 + c) * 4 + s * 16);
    a24 = *reinterpret_cast<const float4*>(a2s + c * NS + 16 * g + s);
  };
  auto wave_scan_combine = [&](const float (&ab)[K][16], float (&bt)[16], float sd, float (&h)[16],
                               float& sd_incl) __attribute__((always_inline)) {
    // QR == 4, distance one sub-chunk: rows 1, 2, 3 take rows 0, 1, 2 (rows 1
    // and 3 from the swap16 pairing, row 2 through swap16 then swap32).
    // Distance QR/2 sub-chunks: rows 2 and 3 take rows 0 and 1 (swap32).
    const bool up1 = q >= 1;
    const bool up2 = r >= 2;
    auto prev_row = [&](float v) __attribute__((always_inline)) {
      float lo, hi, lo2, unused;
      rows_swap16(v, lo, hi);
      rows_swap32(hi, lo2, unused);
      return q == 2 ? lo2 : lo;
    };
#pragma unroll
    for (int S = 0; S < 16; ++S) {
      float a = ab[0][S];
#pragma unroll
      for (int i = 1; i < K; ++i) a *= ab[i][S];
      if constexpr (QR == 4) {
        const float pa = prev_row(a);
        const float pb = prev_row(bt[S]);
        const float nb = __builtin_fmaf(a, pb, bt[S]);
        const float na = pa * a;
        bt[S] = up1 ? nb : bt[S];
        a = up1 ? na : a;
      }
      if constexpr (QR >= 2) {
        float pb, unused;
        rows_swap32(bt[S], pb, unused);
        bt[S] = up2 ? __builtin_fmaf(a, pb, bt[S]) : bt[S];
      }
    }
    float sdi = sd;  // inclusive delta sum over the wave's sub-chunks up to this one
    if constexpr (QR == 4) {
      const float ps = prev_row(sdi);
      sdi = up1 ? ps + sdi : sdi;
    }
    if constexpr (QR >= 2) {
      float ps, unused;
      rows_swap32(sdi, ps, unused);
      sdi = up2 ? ps + sdi : sdi;
    }
    float* const own = agg_b + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
#pragma unroll
    for (int s = 0; s < 16; s += 4)
      *reinterpret_cast<float4*>(own + s * 16) = make_float4(bt[s], bt[s + 1], bt[s + 2], bt[s + 3]);
    if (q == QR - 1 && g == 0) agg_sd[c * SDS + w] = sdi;
    __syncthreads();
    // serial walk over the W wave totals (the last sub-chunk's slot of each
    // wave), leaving each wave's incoming state in wave_in
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      if (pair_valid(k)) {
        int cc, n;
        pair_of(k, cc, n);
        const float a2 = a2s[cc * NS + n];
        float cr = carry[k];
        const int qoff = ((n / 4) * 16 + cc) * 4 + (n % 4);
        const float* ptot = agg_b + (QR - 1) * (N / 4) * 64 + qoff;
        float* pin = wave_in + qoff;
        const float* psd = agg_sd + cc * SDS;
#pragma unroll
        for (int w0 = 0; w0 < W; w0 += 4) {
          float av[4], bb[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            av[u] = fast_exp2(a2 * psd[w0 + u]);
            bb[u] = ptot[(w0 + u) * QR * (N / 4) * 64];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            pin[(w0 + u) * (N / 4) * 64] = cr;
            cr = __builtin_fmaf(av[u], cr, bb[u]);
          }
        }
        carry[k] = cr;
      }
    }
    __syncthreads();
    sd_incl = sdi;
#pragma unroll
    for (int s = 0; s < 16; s += 4) {
      float4 hw4, bi4, a24;
      ws_after_own(s, hw4, bi4, a24);
      const float hws[4] = {hw4.x, hw4.y, hw4.z, hw4.w};
      if constexpr (QR > 1) {
        const float bis[4] = {bi4.x, bi4.y, bi4.z, bi4.w}, a2v[4] = {a24.x, a24.y, a24.z, a24.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // the incoming state is the state after the sub-chunk before
          const float ho = __builtin_fmaf(fast_exp2(a2v[u] * sdi), hws[u], bis[u]);
          float pv;
          if constexpr (QR == 4) {
            pv = prev_row(ho);
          } else {
            float unused;
            rows_swap32(ho, pv, unused);  // rows 2, 3 <- rows 0, 1
          }
          h[s + u] = q == 0 ? hws[u] : pv;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) h[s + u] = hws[u];
      }
    }
  };

  // One tile of T steps starting at step t_tile, with the lane's own x and
  // delta already in xr/dr.  FULL: every step of the tile is valid; otherwise
  // steps at or beyond len are the identity and y there is +0.  When
  // `prefetch` is set, the next tile's x and delta are requested into nxv/ndv
  // before the work of this tile starts, so their latency hides behind it.
  auto tile_body = [&]<bool FULL>(int64_t t_tile, const uint32_t (&xr)[KG], const uint32_t (&dr)[KG],
                                  bool prefetch, uint32_t (&nxv)[KG], uint32_t (&ndv)[KG]) {
    const int64_t left = len - t_tile - j * K;  // valid steps from this lane's first step
    float bv[K], cv[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const bool ok = FULL || i < left;
      const uint32_t sb = static_cast<uint32_t>((t_tile + i) * bc_step);
      bv[i] = ok ? Elem<IO>::template load<0>(rb, off_bc, sb) : 0.0f;
      cv[i] = (ok && !FOLD) ? Elem<IO>::template load<0>(rc, off_bc, sb) : 0.0f;
    }
    if (prefetch) load_xd.template operator()<true>(t_tile + T, nxv, ndv);
    float A2[16];
    {
      const float* pa = a2s + c * NS + 16 * g;
#pragma unroll
      for (int s = 0; s < 16; s += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pa + s);
        A2[s] = v.x;
        A2[s + 1] = v.y;
        A2[s + 2] = v.z;
        A2[s + 3] = v.w;
      }
    }

    // ---- pass 1: discretise, cache Abar, fold the sub-chunk ----
    float ab[K][16];
    float bt[16];
    float dls[K], u[K], xv[K];
    {
      // delta of the lane's own steps first: covers the B/C load latency
      float dlo[KG], uo[KG], xo[KG];
#pragma unroll
      for (int m = 0; m < KG; ++m) {
        float dl = widen(dr[m]) + dbias;
        if constexpr (SOFTPLUS) dl = softplus_f32(dl);
        if constexpr (CLAMP) dl = __builtin_amdgcn_fmed3f(dl, p.dmin, p.dmax);
        if constexpr (!FULL) dl = (g * KG + m < left) ? dl : 0.0f;  // padded step: delta = 0 -> Abar = 1
        xo[m] = widen(xr[m]);
        dlo[m] = dl;
        uo[m] = dl * xo[m];
      }
      share_rows(dlo, dls);
      share_rows(uo, u);
      share_rows(xo, xv);
    }
    float sd = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) sd += dls[i];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float dl = dls[i];
      const float bi = bv[i];
      const float ui = u[i];
      Unroll<0, 16>::run([&]<int S>() {
        ab[i][S] = fast_exp2(dl * A2[S]);
        // the fold starts from zero: the first step's b_total is its b
        bt[S] = (i == 0) ? row_bcast<S>(bi) * ui : __builtin_fmaf(ab[i][S], bt[S], row_bcast<S>(bi) * ui);
      });
    }

    if constexpr (!FOLD) {
#pragma unroll
      for (int i = 0; i < K; ++i) c_s[(j * K + i) * CS + 16 * g + c] = cv[i];
    }
    // Pass 2 needs no state after the sub-chunk's last step, so at dstate 16
    // that step's input term reaches its readout as u (C . B): the row's dot
    // product of the step's B and C (lane c holds state c of both), summed
    // over the 16 lanes with four DPP adds, instead of 16 broadcast products
    // (1.8 % faster; at dstate 32 and 64, and with the wave scan, the extra
    // live value made the compiler spill).
    float cb_last = 0.0f;
    if constexpr (G == 1 && !FOLD && !WSCAN) {
      auto dpp = []<int CTRL>(float v) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
      };
      float t = bv[K - 1] * cv[K - 1];
      t += dpp.template operator()<0xb1>(t);   // quad_perm [1, 0, 3, 2]
      t += dpp.template operator()<0x4e>(t);   // quad_perm [2, 3, 0, 1]
      t += dpp.template operator()<0x141>(t);  // row_half_mirror: the other quad of the half row
      t += dpp.template operator()<0x140>(t);  // row_mirror: the other half row
      cb_last = t;
    }
    float h[16];  // pass 2's state, from the sub-chunk's incoming state
    float sd_incl = 0.0f;  // WSCAN: inclusive delta sum over the wave's sub-chunks up to this one
    if constexpr (WSCAN && !FOLD) {
      wave_scan_combine(ab, bt, sd, h, sd_incl);
    } else {
    {
      float* pb = agg_b + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
#pragma unroll
      for (int s = 0; s < 16; s += 4)
        *reinterpret_cast<float4*>(pb + s * 16) = make_float4(bt[s], bt[s + 1], bt[s + 2], bt[s + 3]);
      if (g == 0) agg_sd[c * SDS + j] = sd;
    }
    __syncthreads();

    // ---- carry walk over the tile's sub-chunks, in time order ----
    // The sub-chunk's decay is a_prod = prod_i exp(delta_i A) = exp2(A log2(e) sum_i delta_i).
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      if (pair_valid(k)) {
        int cc, n;
        pair_of(k, cc, n);
        const float a2 = a2s[cc * NS + n];
        float cr = carry[k];
        float* pbw = agg_b + ((n / 4) * 16 + cc) * 4 + (n % 4);
        const float* psd = agg_sd + cc * SDS;
        // Batches of WB sub-chunks: the LDS reads of a batch are issued
        // together and the decays computed off the carry chain, so the
        // serial part is one FMA and one LDS write per sub-chunk.
        constexpr int WB = kWalkBatch<G>;
        static_assert(WB == 2 || WB % 4 == 0, "delta sums are read as pairs or quads");
#pragma unroll
        for (int j0 = 0; j0 < SUB; j0 += WB) {
          float av[WB], bb[WB];
          if constexpr (WB == 2) {
            const float2 v = *reinterpret_cast<const float2*>(psd + j0);
            av[0] = v.x;
            av[1] = v.y;
          } else {
#pragma unroll
            for (int u = 0; u < WB; u += 4) {
              const float4 v = *reinterpret_cast<const float4*>(psd + j0 + u);
              av[u] = v.x;
              av[u + 1] = v.y;
              av[u + 2] = v.z;
              av[u + 3] = v.w;
            }
          }
#pragma unroll
          for (int u = 0; u < WB; ++u) bb[u] = pbw[(j0 + u) * (N / 4) * 64];
#pragma unroll
          for (int u = 0; u < WB; ++u) {
            if constexpr (FOLD) part_sd[k] += av[u];
            av[u] = fast_exp2(a2 * av[u]);
          }
#pragma unroll
          for (int u = 0; u < WB; ++u) {
            if constexpr (!FOLD) pbw[(j0 + u) * (N / 4) * 64] = cr;
            cr = __builtin_fmaf(av[u], cr, bb[u]);
          }
        }
        carry[k] = cr;
      }
    }
    if constexpr (FOLD) {
      __syncthreads();  // the next tile's pass 1 rewrites the single record buffer
      return;
    }
    if (want_chunks) {
      // The state after sub-chunk jj is the one the walk left for sub-chunk
      // jj + 1 (this lane's own LDS writes), or the carry after the last.
      const int64_t ci0 = (t_begin + t_tile) / p.chunk_len;
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        if (pair_valid(k)) {
          int cc, n;
          pair_of(k, cc, n);
          const float* pbw = agg_b + ((n / 4) * 16 + cc) * 4 + (n % 4);
          for (int jj = clj - 1; jj < SUB; jj += clj)
            store_chunk(ci0 + (jj + 1) / clj - 1, k, jj == SUB - 1 ? carry[k] : pbw[(jj + 1) * (N / 4) * 64]);
        }
      }
    }
    __syncthreads();
    {
      const float* pb = agg_b + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
#pragma unroll
      for (int s = 0; s < 16; s += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pb + s * 16);
        h[s] = v.x;
        h[s + 1] = v.y;
        h[s + 2] = v.z;
        h[s + 3] = v.w;
      }
    }
    }  // serial walk

    // ---- pass 2: states from the incoming state, readout ----
    // y of step i of the sub-chunk, summed over the state groups: the gate,
    // the rounding and the store.  The step's offset from t_tile is soff_step
    // in the scalar offset plus whatever voff adds to the lane's own row.
    auto store_y = [&](int i, int soff_step, uint32_t voff, float yv0) __attribute__((always_inline)) {
      const uint32_t sx = static_cast<uint32_t>((t_tile + soff_step) * xd_step);
      if constexpr (GATE) {
        // y * silu(z), silu(z) = z / (1 + 2^(-z log2 e)); padded steps never load z
        const float zv = (FULL || i < left) ? Elem<IO>::template load<kCached>(rz, voff, sx) : 0.0f;
        yv0 *= zv * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zv * kLog2e));
      }
      if constexpr (FULL) {
        Elem<IO>::store(ry, voff, sx, yv0);
      } else {
        // the tile may run past L; only steps before L exist in y
        const float yv = (i < left) ? yv0 : 0.0f;
        if (i < L - t_tile - j * K) Elem<IO>::store(ry, voff, sx, yv);
      }
    };
    float ysum[K];  // G > 1: this lane's partial y of each step (its 16 states)
#pragma unroll
    for (int i = 0; i < K; ++i) {
      // A fresh name for B so that its broadcasts are not shared with pass 1
      // (sharing would keep 16 broadcast copies live across the carry walk).
      float bi = bv[i];
      asm volatile("" : "+v"(bi));
      const float ui = u[i];
      float ya[2] = {dskip * xv[i], 0.0f};  // two chains: one add per step to join them
      if (G == 1 && !WSCAN && i == K - 1) {
        // the last step: Abar h only, its B u term as u (C . B) (see pass 1)
        Unroll<0, 16>::run([&]<int S>() { h[S] = ab[i][S] * h[S]; });
        ya[1] = ui * cb_last;
      } else {
        Unroll<0, 16>::run([&]<int S>() { h[S] = __builtin_fmaf(ab[i][S], h[S], row_bcast<S>(bi) * ui); });
      }
      {
        const float* crow = c_s + (j * K + i) * CS + 16 * g;
#pragma unroll
        for (int s4 = 0; s4 < 16; s4 += 4) {
          const float4 cq = *reinterpret_cast<const float4*>(crow + s4);
          ya[0] = __builtin_fmaf(cq.x, h[s4], ya[0]);
          ya[1] = __builtin_fmaf(cq.y, h[s4 + 1], ya[1]);
          ya[0] = __builtin_fmaf(cq.z, h[s4 + 2], ya[0]);
          ya[1] = __builtin_fmaf(cq.w, h[s4 + 3], ya[1]);
        }
      }
      ysum[i] = ya[0] + ya[1];
      if constexpr (G == 1) store_y(i, i, off_xd, ysum[i]);
    }
    if constexpr (G > 1 && !FOLD) {  // (the fold kernel has returned above)
      // Reduce-scatter of the K partial sums over the G rows of the sub-chunk:
      // row g ends with the total of steps g, g + G, .. (the steps it stores),
      // added in the order (r0 + r1) + (r2 + r3).  v_permlane16_swap of the
      // partials of steps 2m and 2m + 1 leaves the lower row of each pair
      // holding both rows' step 2m and the upper row both rows' step 2m + 1;
      // at G = 4, v_permlane32_swap then pairs the halves the same way.
      float yown[KG];
      auto swap_pair = [](float& a, float& b, bool halves) __attribute__((always_inline)) {
        if (halves)
          asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
        else
          asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
      };
      float pr[K / 2];
#pragma unroll
      for (int m = 0; m < K / 2; ++m) {
        float a0 = ysum[2 * m], a1 = ysum[2 * m + 1];
        swap_pair(a0, a1, false);
        pr[m] = a0 + a1;
      }
      if constexpr (G == 2) {
#pragma unroll
        for (int m = 0; m < KG; ++m) yown[m] = pr[m];
      } else {
        float q0 = pr[0], q1 = pr[1];
        swap_pair(q0, q1, true);
        yown[0] = q0 + q1;
      }
      const uint32_t off_own = off_xd + static_cast<uint32_t>(g * nd * E);
#pragma unroll
      for (int m = 0; m < KG; ++m) store_y(g + G * m, G * m, off_own, yown[m]);
    }
    if constexpr (WSCAN && !FOLD) {
      // chunk-boundary states: the state after a sub-chunk that ends a chunk
      if (want_chunks && ((j + 1) % clj) == 0) {
        const int64_t ci = (t_begin + t_tile) / p.chunk_len + (j + 1) / clj - 1;
        if (ci < n_chunks) {
          float* dst = p.chunk_states + ((static_cast<int64_t>(b) * n_chunks + ci) * nd + d) * N + 16 * g;
#pragma unroll
          for (int s = 0; s < 16; s += 4) {
            float4 hw4, bi4, a24;
            ws_after_own(s, hw4, bi4, a24);
            dst[s] = __builtin_fmaf(fast_exp2(a24.x * sd_incl), hw4.x, bi4.x);
            dst[s + 1] = __builtin_fmaf(fast_exp2(a24.y * sd_incl), hw4.y, bi4.y);
            dst[s + 2] = __builtin_fmaf(fast_exp2(a24.z * sd_incl), hw4.z, bi4.z);
            dst[s + 3] = __builtin_fmaf(fast_exp2(a24.w * sd_incl), hw4.w, bi4.w);
          }
        }
      }
    }
  };

  __syncthreads();  // a2s is written
  // At dstate 16 the next tile's x and delta are requested before the work of
  // the current tile (1 % faster than loading them at its top).  At 32 and 64
  // the registers they occupy across the tile made the compiler spill (24 and
  // 80 bytes per lane); there each tile loads its own at its top: 1 % and 2 %
  // faster (the fold kernel too, though it does not spill either way).  The
  // wave-scan combine, which needs more registers, never prefetches (dstate
  // 16: 108 -> 56 bytes spilled, 16 % faster).
  constexpr bool kPrefetch = G == 1 && !WSCAN;
  const int64_t nfull = len / T;
  uint32_t xa[KG], da[KG], xn[KG], dn[KG];
  if (kPrefetch && nfull > 0) load_xd.template operator()<true>(0, xa, da);
  for (int64_t tile = 0; tile < nfull; ++tile) {
    if constexpr (!kPrefetch) load_xd.template operator()<true>(tile * T, xa, da);
    tile_body.template operator()<true>(tile * T, xa, da, kPrefetch && tile + 1 < nfull, xn, dn);
    if constexpr (kPrefetch) {
#pragma unroll
      for (int m = 0; m < KG; ++m) {
        xa[m] = xn[m];
        da[m] = dn[m];
      }
    }
  }
  int64_t t_next = nfull * T;
  if (t_next < len) {
    load_xd.template operator()<false>(t_next, xa, da);
    tile_body.template operator()<false>(t_next, xa, da, false, xn, dn);
    t_next += T;
  }
  if constexpr (FOLD) {
    // Part 0 leaves the state entering part 1; a later part its b_total
    // (folded from zero) and the delta sum of each channel over its valid steps.
    float* wb = p.ws + part * ws_block + state_block;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      if (pair_valid(k)) {
        wb[pair_offset(k)] = carry[k];
        int cc, n;
        pair_of(k, cc, n);
        if (part > 0 && n == 0) ws_sd[(static_cast<int64_t>(part - 1) * p.nb + b) * nd + cg * 16 + cc] = part_sd[k];
      }
    }
  } else {
    // Tiles wholly in the padding: the carry is unchanged and y is +0.
    for (; t_next < L; t_next += T) {
      if (want_chunks) {
        const int64_t ci0 = (t_begin + t_next) / p.chunk_len;
#pragma unroll
        for (int k = 0; k < PPL; ++k)
          if (pair_valid(k))
            for (int jj = clj - 1; jj < SUB; jj += clj) store_chunk(ci0 + (jj + 1) / clj - 1, k, carry[k]);
      }
      const int64_t left = L - t_next - j * K;
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if (i < left && (G == 1 || (i % G) == g))
          Elem<IO>::store(ry, off_xd, static_cast<uint32_t>((t_next + i) * xd_step), 0.0f);
      }
    }
    if (p.h_last != nullptr && part == p.n_parts - 1) {
      float* hb = p.h_last + state_block;
#pragma unroll
      for (int k = 0; k < PPL; ++k)
        if (pair_valid(k)) hb[pair_offset(k)] = carry[k];
    }
  }
}

// ---- launch configuration ------------------------------------------------

template <typename IO, int G>
struct Config;
// dstate 16: 8 waves, 4 steps per lane -> 128-step tiles.
template <typename IO>
struct Config<IO, 1> {
  static constexpr int K = 4, W = 8;
};
// dstate 32: 8 waves, 4 steps per lane -> 64-step tiles.
template <typename IO>
struct Config<IO, 2> {
  static constexpr int K = 4, W = 8;
};
// dstate 64: 8 waves, 4 steps per lane -> 32-step tiles.
template <typename IO>
struct Config<IO, 4> {
  static constexpr int K = 4, W = 8;
};

template <typename IO, int G, bool SP, bool CL, bool GATE>
hipError_t launch_flags(const FwdParams& prm, hipStream_t stream) {
  constexpr int K = Config<IO, G>::K, W = Config<IO, G>::W;
  const int64_t groups = static_cast<int64_t>(prm.nb) * prm.n_cg;
  if (prm.n_parts > 1) {
    // The fold of parts 0 .. n_parts-2 must be complete before any part reads
    // its incoming state: same stream, launched first.  The fold never loads
    // z, so it has no gate variant.
    hipLaunchKernelGGL((ssm_fwd_kernel<IO, G, K, W, SP, CL, false, true>),
                       dim3(static_cast<unsigned>(groups * (prm.n_parts - 1))), dim3(64 * W), 0, stream, prm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (prm.wave_scan)
    hipLaunchKernelGGL((ssm_fwd_kernel<IO, G, K, W, SP, CL, GATE, false, true>),
                       dim3(static_cast<unsigned>(groups * prm.n_parts)), dim3(64 * W), 0, stream, prm);
  else
    hipLaunchKernelGGL((ssm_fwd_kernel<IO, G, K, W, SP, CL, GATE, false>),
                       dim3(static_cast<unsigned>(groups * prm.n_parts)), dim3(64 * W), 0, stream, prm);
  return hipGetLastError();
}

template <typename IO, int G, bool SP>
hipError_t launch_sp(const FwdParams& prm, hipStream_t stream) {
  const bool gate = prm.z != nullptr;
  if (prm.clamp)
    return gate ? launch_flags<IO, G, SP, true, true>(prm, stream) : launch_flags<IO, G, SP, true, false>(prm, stream);
  return gate ? launch_flags<IO, G, SP, false, true>(prm, stream) : launch_flags<IO, G, SP, false, false>(prm, stream);
}

template <typename IO, int G>
hipError_t launch(const FwdParams& prm, hipStream_t stream) {
  return prm.softplus ? launch_sp<IO, G, true>(prm, stream) : launch_sp<IO, G, false>(prm, stream);
}

// Steps per time tile of the kernel for state count N (= chunk_len of the
// chunk-boundary states): W waves x (4 / G) sub-chunks per wave x K steps.
template <int G>
constexpr int64_t tile_steps_g = Config<uint16_t, G>::W * (4 / G) * Config<uint16_t, G>::K;
static_assert(tile_steps_g<1> == Config<float, 1>::W * 4 * Config<float, 1>::K, "tile must not depend on io");
// The host accepts chunk lengths that are multiples of 4: every configuration
// uses 4-step sub-chunks.
static_assert(Config<uint16_t, 1>::K == 4 && Config<uint16_t, 2>::K == 4 && Config<uint16_t, 4>::K == 4 &&
                  Config<float, 1>::K == 4 && Config<float, 2>::K == 4 && Config<float, 4>::K == 4,
              "chunk boundaries are sub-chunk boundaries");

int64_t tile_steps(int64_t N) {
  switch (N) {
    case 16:
      return tile_steps_g<1>;
    case 32:
      return tile_steps_g<2>;
    case 64:
      return tile_steps_g<4>;
    default:
      return 0;
  }
}

template <typename IO>
hipError_t launch_io(int G, const FwdParams& prm, hipStream_t stream) {
  switch (G) {
    case 1:
      return launch<IO, 1>(prm, stream);
    case 2:
      return launch<IO, 2>(prm, stream);
    default:
      return launch<IO, 4>(prm, stream);
  }
}

// h_last when there are no time steps: a copy of h0, or zeros.
__global__ void copy_fill_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = (src != nullptr) ? src[i] : 0.0f;
}

// Geometry of a time split into (at most) `parts` parts: whole tiles per part.
struct Split {
  int64_t parts;     // parts actually used (>= 1)
  int64_t part_len;  // steps per part (the last may be shorter)
};

Split split_for(int64_t L, int64_t N, int64_t parts) {
  const int64_t T = tile_steps(N);
  const int64_t n_tiles = L > 0 ? (L + T - 1) / T : 0;
  if (parts <= 1 || n_tiles <= 1) return {1, L};
  const int64_t per = (n_tiles + parts - 1) / parts;
  return {(n_tiles + per - 1) / per, per * T};
}

// Workspace floats of a split: the states entering parts 1 .. P-1 (the first
// directly, the others as b_total of the part before) and the delta sums of
// parts 1 .. P-2.
int64_t split_ws_floats(const Split& sp, int64_t nb, int64_t nd, int64_t N) {
  if (sp.parts <= 1) return 0;
  return (sp.parts - 1) * nb * nd * N + (sp.parts > 2 ? (sp.parts - 2) * nb * nd : 0);
}

}  // namespace

// Scratch of ssm_selective_scan_fwd_noalloc: the time split's carries (the
// workspace of ssm_selective_scan_fwd_ex), in a static array so that the call
// allocates nothing.  Every GPU holds its own copy until the process ends; its
// device address comes from hipGetSymbolAddress at handle creation, since the
// name denotes a host-side stand-in in host code.
static __device__ __align__(256) float scratch[SSM_SCAN_NOALLOC_SCRATCH_BYTES / 4];

namespace {

// Parts for an automatic time split: none while the (row, channel group)
// workgroups alone fill the GPU; otherwise enough parts that the fold of the
// first P-1 parts and the parts themselves each occupy every CU, at most 16
// and at least four tiles per part.
int64_t auto_parts(const ssm_scan_handle_s* h, int64_t nb, int64_t L, int64_t nd, int64_t N) {
  if (N != 16 && N != 32 && N != 64) return 1;
  const int64_t groups = nb * (nd / 16);
  const int64_t slots = static_cast<int64_t>(h->cu_count) * 2;  // resident workgroups: two per CU
  // Split only while whole CUs would sit idle: a workgroup alone on a CU
  // runs about 1.6x faster than one that shares it, and the split adds the
  // fold (about half a forward's work) over all but one part.  Measured at
  // 4096 steps on 256 CUs (ms, unsplit / best split): 128 (row, 16-channel)
  // groups 0.112 / 0.081 (dstate 16), 0.250 / 0.158 (32), 0.527 / 0.318
  // (64); 192 groups 0.113 / 0.113, 0.256 / 0.232, 0.529 / 0.457; 256 groups
  // 0.113 / 0.135, 0.262 / 0.270, 0.539 / 0.548; more groups lose more.
  if (groups <= 0 || 4 * groups > 3 * static_cast<int64_t>(h->cu_count)) return 1;
  // about four workgroups per slot (finer parts balance the tail better:
  // 2.43 ms at 8 parts, 2.34 ms at 16 for one row of 2048 channels x 32768
  // steps, dstate 64), at most 16 parts, and parts of at least four tiles and
  // 512 steps (shorter ones lose to the per-part prologue: 4096 steps, 128
  // groups, dstate 32 and 64: 8 parts 6-8 % faster than 16)
  int64_t parts = (4 * slots + groups - 1) / groups;
  if (parts > 16) parts = 16;
  const int64_t min_part = 4 * tile_steps(N) > 512 ? 4 * tile_steps(N) : 512;
  const int64_t max_by_len = L / min_part;
  if (parts > max_by_len) parts = max_by_len;
  return parts < 1 ? 1 : split_for(L, N, parts).parts;
}

}  // namespace

extern "C" {

int ssm_scan_create(ssm_scan_t* out, int device_ordinal) {
  if (out == nullptr) return SSM_ERR_INVALID_ARG;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess) {
    (void)hipGetLastError();
    return SSM_ERR_NO_DEVICE;
  }
  if (device_ordinal < 0 || device_ordinal >= count) return SSM_ERR_NO_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device_ordinal) != hipSuccess) {
    (void)hipGetLastError();
    return SSM_ERR_HIP;
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return SSM_ERR_UNSUPPORTED;
  // This device's address of the scratch array, taken with the device current.
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device_ordinal) != hipSuccess) {
    (void)hipGetLastError();
    return SSM_ERR_HIP;
  }
  void* scratch_ptr = nullptr;
  const hipError_t sym = hipGetSymbolAddress(&scratch_ptr, HIP_SYMBOL(scratch));
  const hipError_t back = hipSetDevice(prev);
  if (sym != hipSuccess || back != hipSuccess || scratch_ptr == nullptr) {
    (void)hipGetLastError();
    return SSM_ERR_HIP;
  }
  ssm_scan_handle_s* h = new (std::nothrow) ssm_scan_handle_s;
  if (h == nullptr) return SSM_ERR_HIP;
  h->device = device_ordinal;
  h->cu_count = prop.multiProcessorCount;
  h->scratch = static_cast<float*>(scratch_ptr);
  *out = h;
  return SSM_OK;
}

int ssm_scan_destroy(ssm_scan_t handle) {
  delete handle;
  return SSM_OK;
}

const char* ssm_scan_error_string(int code) {
  switch (code) {
    case SSM_OK:
      return "ok";
    case SSM_ERR_INVALID_ARG:
      return "invalid argument (null pointer or handle, negative size, bad flag or clip bounds)";
    case SSM_ERR_UNSUPPORTED:
      return "unsupported (dstate not 16/32/64, dim not a multiple of 16, misaligned pointer, or not gfx950)";
    case SSM_ERR_ALIAS:
      return "an output overlaps an input or the other output";
    case SSM_ERR_HIP:
      return "HIP runtime or launch error";
    case SSM_ERR_NO_DEVICE:
      return "no usable GPU at that ordinal";
    case SSM_ERR_DEVICE_MISMATCH:
      return "the current device is not the handle's device";
    case SSM_ERR_SCRATCH:
      return "the time split asked for needs more than the library's static scratch "
             "(SSM_SCAN_NOALLOC_SCRATCH_BYTES)";
    default:
      return "unknown status code";
  }
}

int64_t ssm_scan_chunk_len(int64_t dstate) { return tile_steps(dstate); }

int32_t ssm_scan_auto_time_parts(ssm_scan_t handle, const ssm_scan_dims* dims) {
  if (handle == nullptr || dims == nullptr || dims->batch < 0 || dims->seqlen < 0 || dims->dim < 0) return 1;
  return static_cast<int32_t>(auto_parts(handle, dims->batch, dims->seqlen, dims->dim, dims->dstate));
}

int64_t ssm_scan_workspace_bytes(const ssm_scan_dims* dims, int32_t time_parts) {
  if (dims == nullptr || time_parts < 0 || dims->batch < 0 || dims->seqlen < 0 || dims->dim < 0) return -1;
  if (tile_steps(dims->dstate) == 0) return -1;
  const Split sp = split_for(dims->seqlen, dims->dstate, time_parts);
  return 4 * split_ws_floats(sp, dims->batch, dims->dim, dims->dstate);
}

}  // extern "C"

namespace {

// The forward behind both entry points.  Checks run in this order: dims,
// sizes and flags; pointers; alignment; aliasing; the handle; the current
// device.  Nothing is enqueued unless all pass.  With use_scratch the time
// split's carries go to the handle's device copy of the static scratch array
// instead of the caller's workspace (whose fields must then be NULL and 0).
int fwd_impl(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B, const void* C,
             const float* D, const int32_t* valid_len, void* y, float* h_last, const ssm_scan_dims* dims,
             const ssm_scan_fwd_extras* extras, void* stream, bool use_scratch) {
  if (dims == nullptr) return SSM_ERR_INVALID_ARG;
  const int64_t nb = dims->batch, L = dims->seqlen, nd = dims->dim, N = dims->dstate;
  if (nb < 0 || L < 0 || nd < 0 || N < 0) return SSM_ERR_INVALID_ARG;
  if (dims->io_dtype != SSM_IO_F32 && dims->io_dtype != SSM_IO_BF16) return SSM_ERR_INVALID_ARG;
  if (dims->delta_softplus != 0 && dims->delta_softplus != 1) return SSM_ERR_INVALID_ARG;
  if (dims->delta_clamp != 0 && dims->delta_clamp != 1) return SSM_ERR_INVALID_ARG;
  if (dims->delta_clamp == 1 && !(dims->delta_min >= 0.0f && dims->delta_min <= dims->delta_max &&
                                  dims->delta_max < __builtin_inff()))
    return SSM_ERR_INVALID_ARG;
  if (N != 16 && N != 32 && N != 64) return SSM_ERR_UNSUPPORTED;
  if (nd % 16 != 0) return SSM_ERR_UNSUPPORTED;
  // Grid and index limits: one workgroup per (row, 16 channels); element
  // indices are 64-bit in the kernel.
  if (nb > 0 && nd > 0 && (nb * (nd / 16) > 0x7fffffffLL || nb > 0x7fffffffLL || nd > 0x7fffffffLL))
    return SSM_ERR_UNSUPPORTED;
  // A batch row of x, delta, y, z, B or C must span fewer than 2^31 bytes (it
  // is addressed through one buffer resource with 32-bit offsets).
  const int64_t esz = dims->io_dtype == SSM_IO_BF16 ? 2 : 4;
  if (L > 0 && L * (N > nd ? N : nd) * esz > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;

  const ssm_scan_fwd_extras none = {nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, 0, SSM_COMBINE_WALK};
  const ssm_scan_fwd_extras& ex = extras ? *extras : none;
  if (ex.combine != SSM_COMBINE_WALK && ex.combine != SSM_COMBINE_WAVE_SCAN) return SSM_ERR_INVALID_ARG;
  // chunk_len: a multiple of the 4-step sub-chunk that divides the tile
  if (ex.chunk_states != nullptr &&
      (ex.chunk_len < 4 || ex.chunk_len % 4 != 0 || tile_steps(N) % ex.chunk_len != 0))
    return SSM_ERR_INVALID_ARG;
  if (ex.time_parts < 0 || ex.workspace_bytes < 0 || (ex.workspace == nullptr && ex.workspace_bytes != 0))
    return SSM_ERR_INVALID_ARG;
  if (use_scratch && (ex.workspace != nullptr || ex.workspace_bytes != 0)) return SSM_ERR_INVALID_ARG;
  const int64_t ws_cap = use_scratch ? static_cast<int64_t>(SSM_SCAN_NOALLOC_SCRATCH_BYTES) : ex.workspace_bytes;
  // An explicit split needs its workspace (or must fit the scratch); the
  // automatic one is skipped when the workspace is missing or too small.
  if (ex.time_parts >= 2) {
    const Split sp = split_for(L, N, ex.time_parts);
    if (4 * split_ws_floats(sp, nb, nd, N) > ws_cap) return use_scratch ? SSM_ERR_SCRATCH : SSM_ERR_INVALID_ARG;
  }

  const bool empty = (nb == 0 || nd == 0);
  const size_t e = static_cast<size_t>(esz);
  const size_t n_xd = static_cast<size_t>(nb) * L * nd, n_bc = static_cast<size_t>(nb) * L * N;
  const size_t n_state = static_cast<size_t>(nb) * nd * N;
  const int64_t cl = ex.chunk_states != nullptr ? ex.chunk_len : tile_steps(N);
  const size_t n_chunks = (L > 0 && cl > 0) ? static_cast<size_t>((L + cl - 1) / cl) : 0;
  if (!empty) {
    if (A_log == nullptr) return SSM_ERR_INVALID_ARG;
    if (L > 0 && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || y == nullptr))
      return SSM_ERR_INVALID_ARG;
    if (!aligned(x, e) || !aligned(delta, e) || !aligned(B, e) || !aligned(C, e) || !aligned(y, e) ||
        !aligned(ex.z, e) || !aligned(A_log, 4) || !aligned(D, 4) || !aligned(valid_len, 4) || !aligned(h_last, 4) ||
        !aligned(ex.h0, 4) || !aligned(ex.delta_bias, 4) || !aligned(ex.chunk_states, 4) ||
        !aligned(ex.workspace, 4))
      return SSM_ERR_UNSUPPORTED;
    const size_t by = L > 0 ? n_xd * e : 0, bh = h_last ? n_state * 4 : 0;
    const size_t bcs = ex.chunk_states ? n_chunks * n_state * 4 : 0;
    const void* ins[] = {x, delta, B, C, A_log, D, valid_len, L > 0 ? ex.z : nullptr, ex.h0, ex.delta_bias};
    const size_t ins_n[] = {n_xd * e, n_xd * e, n_bc * e, n_bc * e, static_cast<size_t>(nd) * N * 4,
                            D ? static_cast<size_t>(nd) * 4 : 0, valid_len ? static_cast<size_t>(nb) * 4 : 0,
                            ex.z ? n_xd * e : 0, ex.h0 ? n_state * 4 : 0, ex.delta_bias ? static_cast<size_t>(nd) * 4 : 0};
    for (int k = 0; k < 10; ++k) {
      // h0 may be h_last itself: unsplit, each state element is read before
      // the same thread overwrites it (a split runs unsplit then, below).
      const bool h0_in_place = (ins[k] == ex.h0 && ex.h0 != nullptr && static_cast<const void*>(h_last) == ex.h0);
      if (overlaps(y, by, ins[k], ins_n[k]) || overlaps(ex.chunk_states, bcs, ins[k], ins_n[k]))
        return SSM_ERR_ALIAS;
      if (!h0_in_place && overlaps(h_last, bh, ins[k], ins_n[k])) return SSM_ERR_ALIAS;
    }
    if (overlaps(y, by, h_last, bh) || overlaps(y, by, ex.chunk_states, bcs) ||
        overlaps(h_last, bh, ex.chunk_states, bcs))
      return SSM_ERR_ALIAS;
    // The workspace is written by the library: it may overlap nothing else.
    const size_t bw = static_cast<size_t>(ex.workspace_bytes);
    for (int k = 0; k < 10; ++k)
      if (overlaps(ex.workspace, bw, ins[k], ins_n[k])) return SSM_ERR_ALIAS;
    if (overlaps(ex.workspace, bw, y, by) || overlaps(ex.workspace, bw, h_last, bh) ||
        overlaps(ex.workspace, bw, ex.chunk_states, bcs))
      return SSM_ERR_ALIAS;
  }
  if (handle == nullptr) return SSM_ERR_INVALID_ARG;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return SSM_ERR_HIP;
  }
  if (cur != handle->device) return SSM_ERR_DEVICE_MISMATCH;
  if (empty) return SSM_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L == 0) {
    // No steps: the final state is the initial one.
    if (h_last == nullptr) return SSM_OK;
    const int64_t n = nb * nd * N;
    if (ex.h0 != nullptr) {
      if (ex.h0 == h_last) return SSM_OK;
      hipLaunchKernelGGL(copy_fill_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, h_last,
                         ex.h0, n);
    } else {
      hipLaunchKernelGGL(copy_fill_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, h_last,
                         static_cast<const float*>(nullptr), n);
    }
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }

  FwdParams prm;
  prm.x = x;
  prm.delta = delta;
  prm.A_log = A_log;
  prm.B = B;
  prm.C = C;
  prm.D = D;
  prm.valid_len = valid_len;
  prm.y = y;
  prm.h_last = h_last;
  prm.h0 = ex.h0;
  prm.delta_bias = ex.delta_bias;
  prm.z = ex.z;
  prm.chunk_states = ex.chunk_states;
  prm.chunk_len = ex.chunk_states != nullptr ? ex.chunk_len : tile_steps(N);
  prm.L = L;
  prm.nb = static_cast<int32_t>(nb);
  prm.nd = static_cast<int32_t>(nd);
  prm.n_cg = static_cast<int32_t>(nd / 16);
  prm.softplus = dims->delta_softplus;
  prm.clamp = dims->delta_clamp;
  prm.dmin = dims->delta_min;
  prm.dmax = dims->delta_max;
  prm.wave_scan = ex.combine == SSM_COMBINE_WAVE_SCAN;
  prm.pair_rows = 0;
  int64_t parts = ex.time_parts;
  if (parts == 0) {
    parts = auto_parts(handle, nb, L, nd, N);
    if (parts >= 2 && 4 * split_ws_floats(split_for(L, N, parts), nb, nd, N) > ws_cap) parts = 1;
  }
  // In place (h0 == h_last) the scan runs unsplit: split, the first part's
  // workgroups would read h0 while the last part's, in the same launch, write
  // h_last over it.
  if (ex.h0 != nullptr && static_cast<const void*>(ex.h0) == static_cast<const void*>(h_last)) parts = 1;
  const Split sp = split_for(L, N, parts);
  if (static_cast<int64_t>(nb) * (nd / 16) * sp.parts > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;
  prm.pair_rows = use_length_pairing(valid_len, sp.parts, nb, nd / 16, handle->cu_count) ? 1 : 0;
  prm.ws = use_scratch ? handle->scratch : static_cast<float*>(ex.workspace);
  prm.part_len = sp.part_len;
  prm.n_parts = static_cast<int32_t>(sp.parts);
  const int G = static_cast<int>(N / 16);
  const hipError_t err =
      dims->io_dtype == SSM_IO_BF16 ? launch_io<uint16_t>(G, prm, s) : launch_io<float>(G, prm, s);
  return err == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_selective_scan_fwd_ex(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B,
                              const void* C, const float* D, const int32_t* valid_len, void* y, float* h_last,
                              const ssm_scan_dims* dims, const ssm_scan_fwd_extras* extras, void* stream) {
  return fwd_impl(handle, x, delta, A_log, B, C, D, valid_len, y, h_last, dims, extras, stream, false);
}

int ssm_selective_scan_fwd_noalloc(ssm_scan_t handle, const void* x, const void* delta, const float* A_log,
                                   const void* B, const void* C, const float* D, const int32_t* valid_len, void* y,
                                   float* h_last, const ssm_scan_dims* dims, const ssm_scan_fwd_extras* extras,
                                   void* stream) {
  return fwd_impl(handle, x, delta, A_log, B, C, D, valid_len, y, h_last, dims, extras, stream, true);
}

int ssm_selective_scan_fwd(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B,
                           const void* C, const float* D, const int32_t* valid_len, void* y, float* h_last,
                           const ssm_scan_dims* dims, void* stream) {
  return fwd_impl(handle, x, delta, A_log, B, C, D, valid_len, y, h_last, dims, nullptr, stream, false);
}

}  // extern "C"
