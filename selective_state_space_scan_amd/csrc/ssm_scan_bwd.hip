// Backward of the fused selective-scan forward for MI355X (gfx950) and its C
// ABI entry points.
//
// With the loss sum(dy * y) + sum(dh_last * h_last) and A = -exp(A_log), the
// adjoint g_t of the state after step t obeys the reverse recurrence
//     g_t = dh_last [t = last valid step] + dyp_t * C_t + Abar_{t+1} g_{t+1},
// dyp_t = dy_t * silu(z_t) with the gate (else dy_t).  Written for mu_t, the
// adjoint of the state before step t, it is the affine map
//     mu_t = Abar_t * (dyp_t * C_t + mu_{t+1})
// with per-step coefficients, so it composes over sub-chunks exactly like the
// forward pair (Abar, b) and runs in reverse with the same fold / carry walk /
// rescan structure as the forward kernel (the associative scan of the pwwt.cn
// article, sections 2.1 and 3.1, applied to flipped time; the forward states it
// needs are recomputed from the chunk-boundary states the forward saved, its
// section 3.4).  Per step and state (g = mu_{t+1} + dyp_t C_t):
//     dC[t,n] += dyp_t h_t            dB[t,n] += g Delta_t x_t    (sums over channels)
//     dx_t = dyp_t D + Delta_t sum_n g B_t          dD += dyp_t x_t
//     dDelta_t = x_t sum_n g B_t + sum_n g h_{t-1} Abar_t A
//     dA[n] += g h_{t-1} Abar_t Delta_t,  dA_log = dA * A
//     dDelta_raw = dDelta * [clip passes] * sigmoid(raw + bias),  dbias = sum dDelta_raw
//     dz_t = dy_t (C_t . h_t + D x_t) silu'(z_t),  dh0 = mu_0.
//
// Work mapping (one workgroup = one batch row x 16 channels, as in the
// forward): a lane owns one channel, 16 states and K = 2 consecutive steps of
// a tile; tiles are visited from the last to the first and the adjoint carry
// stays in a register from tile to tile.  Per tile:
//  * pass 1: Delta, u = Delta x, Abar (cached, 2 x 16 VGPRs), the forward fold
//    b_total and the reverse fold m = Abar_0 (c_0 + Abar_1 c_1), c = dyp C, to
//    LDS;
//  * walks (one lane per (channel, state)): the forward walk from the tile's
//    saved start state leaves each sub-chunk's incoming state in LDS; the
//    reverse walk from the adjoint carry leaves each sub-chunk's mu_{end+1};
//  * pass 2: the lane rebuilds h over its K steps and runs the adjoint back
//    over them, producing dx, dDelta_raw, dz, dA; the per-(step, state)
//    contributions to dB and dC are summed over the 16 channels by a DPP
//    reduce-scatter across the lanes and written as one partial per channel
//    group.
// At dstate 32 and 64 the state-group rows of a sub-chunk split its
// per-(step, channel) work (loads, softplus, gate) and reduce-scatter their
// per-step sums over states, exchanging values with v_permlane16/32_swap.
// With a time split, a fold kernel first folds the adjoint of every part but
// the first from zero, over 8-step sub-chunks (it keeps no per-step state).
// A last kernel sums the partials over channel groups (dB, dC) and over
// batch rows and parts (dA_log, dD, dbias) in a fixed order, so the result is
// deterministic.
//
// All arithmetic is fp32.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "ssm_internal.h"
#include "ssm_scan.h"

namespace {

struct BwdParams {
  const void* x;
  const void* delta;
  const float* A_log;
  const void* B;
  const void* C;
  const float* D;
  const int32_t* valid_len;
  const float* h0;
  const float* delta_bias;
  const void* z;
  const float* chunk_states;  // [nb, ceil(L / T), nd, N]: the state after every tile of T steps
  const void* dy;
  const float* dh_last;
  void* dx;
  void* ddelta;
  void* dz;
  float* dh0;
  float* ws_dB;  // [n_cg, nb, L, N] partial sums over the 16 channels of a group
  float* ws_dC;
  float* ws_dA;  // [n_parts, nb, nd, N]
  float* ws_dD;  // [n_parts, nb, nd]
  float* ws_db;  // [n_parts, nb, nd]
  // Time split (small batches): parts of part_len steps (whole tiles).  The
  // fold kernel leaves, for parts 1 .. n_parts-1, the adjoint folded from zero
  // over the part (ws_M [n_parts-1, nb, nd, N]) and its delta sums (ws_S
  // [n_parts-1, nb, nd]); part p then starts from dh_last carried back through
  // parts n_parts-1 .. p+1.
  float* ws_M;
  float* ws_S;
  int64_t part_len;
  int32_t n_parts;
  int64_t L;
  int64_t n_chunks;  // chunk states per row (chunks of the 4-wave tile)
  int32_t nb;
  int32_t nd;
  int32_t n_cg;
  int32_t pair_rows;  // rows of different lengths: pair the longest with the shortest on each CU
  int32_t clamp;
  float dmin;
  float dmax;
};

constexpr int kBwdK = 2;  // steps per lane and sub-chunk
// The fold kernel of a time split keeps no per-step state (no Abar cache, no
// pass 2), so its sub-chunks are longer: the walk's exp and FMA chain per
// (pair, sub-chunk) is then spread over 8 steps instead of 2.
constexpr int kBwdFoldK = 8;
// Waves per workgroup: 4 when the grid fills the GPU (two workgroups share a
// CU and cover each other's barriers), 8 for small grids (more waves per
// (row, channel group)).  The chunk length of the saved states is the 4-wave
// tile; an 8-wave tile reads every other chunk state.
constexpr int kBwdW = 4;

template <int G>
constexpr int64_t bwd_tile_g = kBwdW * (4 / G) * kBwdK;

int64_t bwd_tile(int64_t N) {
  switch (N) {
    case 16:
      return bwd_tile_g<1>;
    case 32:
      return bwd_tile_g<2>;
    case 64:
      return bwd_tile_g<4>;
    default:
      return 0;
  }
}

__device__ __forceinline__ float sigmoid_f32(float v) { return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e)); }

// softplus(v) (as softplus_f32) and its derivative sigmoid(v) from one exp:
// with e = exp(-|v|) and w = 1 + e, sigmoid(v) = 1 / w for v >= 0 and e / w
// below.
__device__ __forceinline__ float softplus_sigmoid_f32(float v, float& sig) {
  const float e = fast_exp2(-__builtin_fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  const float rw = __builtin_amdgcn_rcpf(w);
  sig = (v >= 0.0f) ? rw : e * rw;
  return __builtin_fmaxf(v, 0.0f) + log1p_of_exp_term(e, w);
}

// Reduce-scatter over the 16 lanes of a DPP row: every lane holds v[0..15];
// lane c of the row gets the sum over the row's 16 lanes of their v[c].  A
// four-level butterfly: at each level a lane keeps the half of its values
// whose index bit matches its own lane bit and adds its partner's copy of
// that half, the partner being lane c ^ 8 (row_ror:8), the mirror lane within
// the 8-lane half (row_half_mirror; differs in bit 2), then c ^ 2 and c ^ 1
// (quad_perm).  The first two levels pick the kept half per group of four
// lanes with bank_mask, two masked DPP adds writing complementary lanes of
// one register, so they need no selects; the last two select with
// v_cndmask.  The order of the additions depends only on lane positions.
// The leading s_nop covers the DPP hazards as in dot16_row_bcast; the early
// clobbers keep the outputs out of the inputs' registers, since the first
// masked add of each pair writes its output before the block has read every
// input.  `c` is the lane's position in its row.
__device__ __forceinline__ float row_reduce_scatter16(const float (&v)[16], int c) {
  float h[8], q[4];
  asm volatile(
      "s_nop 4\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %16, %16 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %17, %17 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %18, %18 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %19, %19 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %4, %20, %20 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %5, %21, %21 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %6, %22, %22 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %7, %23, %23 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(h[4]), "=&v"(h[5]), "=&v"(h[6]), "=&v"(h[7])
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]), "v"(v[8]),
        "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
  asm volatile(
      "s_nop 4\n\t"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3])
      : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]), "v"(h[6]), "v"(h[7]));
  // c ^ 2: keep q[0..1] (bit 1 clear) or q[2..3]
  const bool b1 = (c & 2) != 0, b0 = (c & 1) != 0;
  auto xchg = []<int CTRL>(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
  };
  constexpr int kXor2 = 0x4e, kXor1 = 0xb1;  // quad_perm [2,3,0,1] and [1,0,3,2]
  const float r0 = (b1 ? q[2] : q[0]) + xchg.template operator()<kXor2>(b1 ? q[0] : q[2]);
  const float r1 = (b1 ? q[3] : q[1]) + xchg.template operator()<kXor2>(b1 ? q[1] : q[3]);
  // c ^ 1
  return (b0 ? r1 : r0) + xchg.template operator()<kXor1>(b0 ? r0 : r1);
}

// FOLD: the fold kernel of the time split (pass 1 and the reverse walk only,
// over parts 1 .. n_parts-1).  Otherwise the backward over every part.
template <typename IO, int G, int W, bool SOFTPLUS, bool CLAMP, bool GATE, bool FOLD>
__global__ __launch_bounds__(64 * W, 2) void ssm_bwd_kernel(BwdParams p) {
  constexpr int K = FOLD ? kBwdFoldK : kBwdK;
  constexpr int CS = W / kBwdW;  // saved chunks per tile (not used by the fold)
  constexpr int N = 16 * G;
  constexpr int QR = 4 / G;
  constexpr int SUB = W * QR;  // sub-chunks per tile
  constexpr int T = SUB * K;   // steps per tile
  constexpr int NS = N + 4;
  constexpr int SDS = SUB + 4;
  constexpr int AGG = SUB * 16 * N;
  constexpr int PAIRS = 16 * N;
  constexpr int NT = 64 * W;
  constexpr int PPL = (PAIRS + NT - 1) / NT;
  constexpr int E = Elem<IO>::kBytes;
  static_assert(SUB % 4 == 0, "sub-chunk records are read as quads");
  static_assert(SUB * G * 16 == NT, "one lane per (sub-chunk, state group, channel)");

  // Sub-chunk records, float4 quads as in the forward: index
  // ((j * N/4 + n/4) * 16 + c) * 4 + n%4.  agg_b: forward b_total, then the
  // state entering the sub-chunk; agg_m: reverse fold m, then mu at the
  // sub-chunk's end.  After the last tile agg_b stages the dA sums.
  __shared__ __attribute__((aligned(16))) float agg_b[AGG];
  __shared__ __attribute__((aligned(16))) float agg_m[AGG];
  __shared__ __attribute__((aligned(16))) float agg_sd[16 * SDS];
  __shared__ __attribute__((aligned(16))) float a2s[16 * NS];
  __shared__ float red[2][NT];  // end of kernel: dD and dbias per lane

  const int64_t groups = static_cast<int64_t>(p.nb) * p.n_cg;
  const int64_t total = groups * (FOLD ? p.n_parts - 1 : p.n_parts);
  const int64_t bid = blockIdx.x;
  const int64_t per_xcd = total / 8;
  const int64_t logical = (bid < per_xcd * 8) ? (bid % 8) * per_xcd + bid / 8 : bid;
  const int part = static_cast<int>(logical / groups) + (FOLD ? 1 : 0);
  int b = static_cast<int>((logical % groups) / p.n_cg);
  int cg = static_cast<int>(logical % p.n_cg);
  // rows of different lengths: the longest row shares its CUs with the shortest
  __shared__ int32_t row_lens[64], row_order[64];
  if (!FOLD && p.pair_rows) length_paired_row(bid, groups, p.n_cg, p.nb, p.L, p.valid_len, row_lens, row_order, b, cg);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int r = lane >> 4;
  const int c = lane & 15;
  const int q = r / G;
  const int g = r % G;
  const int j = w * QR + q;
  const int d = cg * 16 + c;
  const int nd = p.nd;
  // This workgroup's steps [t_begin, t_begin + L); below, step indices are
  // relative to t_begin.
  const int64_t t_begin = part * p.part_len;
  const int64_t L = (p.L - t_begin < p.part_len) ? p.L - t_begin : p.part_len;
  int64_t len = p.L;
  if (p.valid_len != nullptr) {
    const int64_t v = p.valid_len[b];
    len = v < 0 ? 0 : (v > p.L ? p.L : v);
  }
  len -= t_begin;
  len = len < 0 ? 0 : (len > L ? L : len);

  for (int k = tid; k < 16 * N; k += NT) {
    const int cc = k / N, n = k % N;
    a2s[cc * NS + n] = -expf(p.A_log[static_cast<int64_t>(cg * 16 + cc) * N + n]) * kLog2e;
  }
  const float dskip = (p.D != nullptr) ? p.D[d] : 0.0f;
  const float dbias = (p.delta_bias != nullptr) ? p.delta_bias[d] : 0.0f;

  // The walk lane's (channel, state) pair k: each group of 64 pairs is 16
  // channels x 4 states, state fastest, so that a wave's lanes touch 64
  // consecutive words of a record slot (with the channel fastest, channels c
  // and c + 8 shared an LDS bank: 0.3 / 1.3 / 4.1 % slower at dstate
  // 16 / 32 / 64).
  auto pair_of = [&](int k, int& cc, int& n) {
    const int pr = tid + k * NT;
    cc = (pr & 63) >> 2;
    n = 4 * (pr >> 6) + (pr & 3);
  };
  auto pair_valid = [&](int k) { return PAIRS % NT == 0 || tid + k * NT < PAIRS; };
  auto pair_offset = [&](int k) {
    int cc, n;
    pair_of(k, cc, n);
    return static_cast<uint32_t>(cc * N + n);
  };
  const int64_t state_block = (static_cast<int64_t>(b) * nd + cg * 16) * N;
  const int64_t n_tiles = (L + T - 1) / T;
  const int64_t tile0 = t_begin / T;  // global index of the part's first tile
  const int64_t sblock = static_cast<int64_t>(p.nb) * nd * N;

  // The adjoint carry (mu entering the current tile from the future) and the
  // per-pair dA accumulator, held by the walk lanes.  A part other than the
  // last starts from dh_last carried back through the later parts' folds.
  float mu_carry[PPL], dA_acc[PPL], part_sd[PPL];
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    dA_acc[k] = 0.0f;
    part_sd[k] = 0.0f;
    mu_carry[k] = 0.0f;
    if (!FOLD && pair_valid(k)) {
      float mu = (p.dh_last != nullptr) ? p.dh_last[state_block + pair_offset(k)] : 0.0f;
      if (part < p.n_parts - 1) {
        int cc, n;
        pair_of(k, cc, n);
        const float a2 = -expf(p.A_log[static_cast<int64_t>(cg * 16 + cc) * N + n]) * kLog2e;
        for (int qp = p.n_parts - 1; qp > part; --qp) {
          const float sdq = p.ws_S[(static_cast<int64_t>(qp - 1) * p.nb + b) * nd + cg * 16 + cc];
          mu = __builtin_fmaf(fast_exp2(a2 * sdq), mu, p.ws_M[(qp - 1) * sblock + state_block + pair_offset(k)]);
        }
      }
      mu_carry[k] = mu;
    }
  }
  float dD_acc = 0.0f, db_acc = 0.0f;  // this lane's steps, channel d (counted once per (t, d))
  float dAl[16];  // this lane's dA contributions for its 16 states, over all tiles
#pragma unroll
  for (int s = 0; s < 16; ++s) dAl[s] = 0.0f;

  const int64_t xd_step = static_cast<int64_t>(nd) * E;
  const int64_t bc_step = static_cast<int64_t>(N) * E;
  const int64_t xd_base = (b * p.L + t_begin) * xd_step, bc_base = (b * p.L + t_begin) * bc_step;
  const int64_t xd_row = L * xd_step, bc_row = L * bc_step;
  const rsrc_t rx = make_rsrc(static_cast<const char*>(p.x) + xd_base, xd_row);
  const rsrc_t rd = make_rsrc(static_cast<const char*>(p.delta) + xd_base, xd_row);
  const rsrc_t rdy = make_rsrc(static_cast<const char*>(p.dy) + xd_base, xd_row);
  const rsrc_t rz = make_rsrc(GATE ? static_cast<const char*>(p.z) + xd_base : nullptr, GATE ? xd_row : 0);
  const rsrc_t rdx = make_rsrc(FOLD ? nullptr : static_cast<char*>(p.dx) + xd_base, FOLD ? 0 : xd_row);
  const rsrc_t rdd = make_rsrc(FOLD ? nullptr : static_cast<char*>(p.ddelta) + xd_base, FOLD ? 0 : xd_row);
  const rsrc_t rdz =
      make_rsrc(GATE && !FOLD ? static_cast<char*>(p.dz) + xd_base : nullptr, GATE && !FOLD ? xd_row : 0);
  const rsrc_t rb = make_rsrc(static_cast<const char*>(p.B) + bc_base, bc_row);
  const rsrc_t rc = make_rsrc(static_cast<const char*>(p.C) + bc_base, bc_row);
  const uint32_t off_xd = static_cast<uint32_t>((j * K * nd + d) * E);
  // The 2 (dstate 32) or 4 (dstate 64) state-group rows of a sub-chunk share
  // its steps: a lane loads x, delta, dy, z and runs softplus, the clip and
  // the gate only for its own steps, and the rows exchange the results with
  // v_permlane16_swap (and v_permlane32_swap).  With K = 2 steps row r takes
  // step r % 2 (rows [0, 0, 2, 2] hold step 0 after the swap, rows
  // [1, 1, 3, 3] step 1); in the fold (K = 8) row g takes steps g*KS ..
  // g*KS + KS-1.  At dstate 16 a lane has all its steps.
  constexpr int KS = G == 1 ? K : (FOLD ? K / G : 1);  // steps a lane discretises
  static_assert(FOLD || K == 2, "the row exchange pairs rows 2q and 2q + 1 over two steps");
  static_assert(!FOLD || K % G == 0, "the fold's rows split a sub-chunk's steps evenly");
  auto own_step = [&](int m) { return G == 1 ? m : (FOLD ? g * KS + m : (r & 1)); };
  const uint32_t off_xd_own = off_xd + static_cast<uint32_t>((G == 1 ? 0 : (FOLD ? g * KS : (r & 1))) * nd * E);
  auto share_rows = [](const float (&own)[KS], float (&all)[K]) __attribute__((always_inline)) {
    if constexpr (G == 1) {
#pragma unroll
      for (int i = 0; i < K; ++i) all[i] = own[i];
    } else if constexpr (!FOLD) {
      rows_swap16(own[0], all[0], all[1]);
    } else if constexpr (G == 2) {
#pragma unroll
      for (int m = 0; m < KS; ++m) rows_swap16(own[m], all[m], all[KS + m]);  // rows 2q and 2q + 1
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        float lo, hi;
        rows_swap16(own[m], lo, hi);  // rows [0, 0, 2, 2] and [1, 1, 3, 3]
        rows_swap32(lo, all[m], all[2 * KS + m]);
        rows_swap32(hi, all[KS + m], all[3 * KS + m]);
      }
    }
  };
  const uint32_t off_bc = static_cast<uint32_t>((j * K * N + 16 * g + c) * E);
  // dB / dC partials of this channel group: [n_cg, nb, L, N], from the part's first step
  float* const wdB = p.ws_dB + ((static_cast<int64_t>(cg) * p.nb + b) * p.L + t_begin) * N;
  float* const wdC = p.ws_dC + ((static_cast<int64_t>(cg) * p.nb + b) * p.L + t_begin) * N;

  __syncthreads();  // a2s is written

  // The state entering tile kt (h0, or the chunk state the forward saved) is
  // loaded at the top of the tile, so that its latency hides behind pass 1.
  // With four pairs per thread (dstate 64) that just fits in 256 VGPRs (the
  // gated variants spill a few dwords) and is still 9 % faster than loading
  // it where the walk needs it.  (Loading it a whole tile ahead costs a
  // register copy at the loop's end, which waits for every outstanding memory
  // operation, stores included.)
  constexpr bool kAhead = PPL <= 4;
  auto load_h_in = [&](int64_t kt, int k) -> float {
    const int64_t gt = tile0 + kt;
    if (gt == 0) return (p.h0 != nullptr) ? p.h0[state_block + pair_offset(k)] : 0.0f;
    return p.chunk_states[((static_cast<int64_t>(b) * p.n_chunks + gt * CS - 1) * nd + cg * 16) * N +
                          pair_offset(k)];
  };

  for (int64_t kt = n_tiles - 1; kt >= 0; --kt) {
    const int64_t t_tile = kt * T;
    const int64_t left = len - t_tile - j * K;  // valid steps from this lane's first step
    if (len <= t_tile) {
      // A tile wholly in the padding: zero gradients, the adjoint passes through.
      if constexpr (FOLD) continue;
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if (j * K + i < L - t_tile && (G == 1 || (i % G) == g)) {
          const uint32_t sx = static_cast<uint32_t>((t_tile + i) * xd_step);
          Elem<IO>::store(rdx, off_xd, sx, 0.0f);
          Elem<IO>::store(rdd, off_xd, sx, 0.0f);
          if constexpr (GATE) Elem<IO>::store(rdz, off_xd, sx, 0.0f);
        }
      }
      continue;
    }

    // ---- loads ----
    float h_in[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) h_in[k] = (kAhead && !FOLD && pair_valid(k)) ? load_h_in(kt, k) : 0.0f;
    // A tile wholly inside the valid length (every one but the last) loads
    // without per-lane conditions, so that its loads issue together instead
    // of one masked branch (and one wait) per load.
    const bool full = t_tile + T <= len;  // uniform over the workgroup
    // x, delta, dy, z: the lane's own steps only (KS of them, see own_step)
    float xo[KS], dlr[KS], dyo[KS], zo[KS], bv[K], cv[K];
    if (full) {
      // (B and C first: a different order from the masked loads below keeps
      // the compiler from merging the two paths' last loads into one block)
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const uint32_t sb = static_cast<uint32_t>((t_tile + i) * bc_step);
        cv[i] = Elem<IO>::template load<0>(rc, off_bc, sb);
        bv[i] = !FOLD ? Elem<IO>::template load<0>(rb, off_bc, sb) : 0.0f;
      }
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const uint32_t sx = static_cast<uint32_t>((t_tile + m) * xd_step);
        // the fold needs neither x nor B (only the adjoint input dyp * C)
        xo[m] = !FOLD ? Elem<IO>::template load<kCached>(rx, off_xd_own, sx) : 0.0f;
        dlr[m] = Elem<IO>::template load<kCached>(rd, off_xd_own, sx);
        dyo[m] = Elem<IO>::template load<kCached>(rdy, off_xd_own, sx);
        zo[m] = GATE ? Elem<IO>::template load<kCached>(rz, off_xd_own, sx) : 0.0f;
      }
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const bool ok = own_step(m) < left;
        const uint32_t sx = static_cast<uint32_t>((t_tile + m) * xd_step);
        xo[m] = (ok && !FOLD) ? Elem<IO>::template load<kCached>(rx, off_xd_own, sx) : 0.0f;
        dlr[m] = ok ? Elem<IO>::template load<kCached>(rd, off_xd_own, sx) : 0.0f;
        dyo[m] = ok ? Elem<IO>::template load<kCached>(rdy, off_xd_own, sx) : 0.0f;
        zo[m] = (GATE && ok) ? Elem<IO>::template load<kCached>(rz, off_xd_own, sx) : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const bool ok = i < left;
        const uint32_t sb = static_cast<uint32_t>((t_tile + i) * bc_step);
        bv[i] = (ok && !FOLD) ? Elem<IO>::template load<0>(rb, off_bc, sb) : 0.0f;
        cv[i] = ok ? Elem<IO>::template load<0>(rc, off_bc, sb) : 0.0f;
      }
    }
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

    // ---- pass 1 ----
    float dl[K], fac[K], u[K], dyp[K], sg_z[K], xv[K], dyv[K], zv[K];
    {
      float dlo[KS], faco[KS], uo[KS], dypo[KS], sgo[KS];
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const bool ok = own_step(m) < left;
        const float raw = dlr[m] + dbias;
        float v = raw, f = 1.0f;
        if constexpr (SOFTPLUS) {
          v = softplus_sigmoid_f32(raw, f);
        }
        if constexpr (CLAMP) {
          f = (v >= p.dmin && v <= p.dmax) ? f : 0.0f;
          v = __builtin_amdgcn_fmed3f(v, p.dmin, p.dmax);
        }
        dlo[m] = ok ? v : 0.0f;
        faco[m] = ok ? f : 0.0f;
        uo[m] = dlo[m] * xo[m];
        if constexpr (GATE) {
          sgo[m] = sigmoid_f32(zo[m]);
          dypo[m] = dyo[m] * zo[m] * sgo[m];
        } else {
          sgo[m] = 0.0f;
          dypo[m] = dyo[m];
        }
      }
      share_rows(dlo, dl);
      share_rows(faco, fac);
      share_rows(uo, u);
      share_rows(dypo, dyp);
      if constexpr (!FOLD) share_rows(xo, xv);
      if constexpr (GATE) {
        share_rows(sgo, sg_z);
        share_rows(dyo, dyv);
        share_rows(zo, zv);
      } else {
#pragma unroll
        for (int i = 0; i < K; ++i) {
          sg_z[i] = 0.0f;
          dyv[i] = dyp[i];
          zv[i] = 0.0f;
        }
      }
      if constexpr (FOLD) {
#pragma unroll
        for (int i = 0; i < K; ++i) xv[i] = 0.0f;
      }
    }
    float sd = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) sd += dl[i];
    // Abar and the input terms B u of both steps stay in registers for pass 2
    // (the fold kernel, which has no pass 2, leaves ab, bu and cy unused)
    float ab[K][16], bu[K][16];
    float bt[16], mm[16];
    // c = dyp C (pass 2 adds the same terms to the adjoint)
    float cy[K][16];
    if constexpr (FOLD) {
      // the sub-chunk's reverse fold from zero, m = Abar_0 (c_0 + Abar_1 (c_1
      // + .. Abar_{K-1} c_{K-1})), from the last step back with one FMA per
      // step: p = c_{K-1}, p = Abar_i p + c_{i-1}, m = Abar_0 p
      float pp[16];
      {
        const float ck = cv[K - 1], yk = dyp[K - 1];
        Unroll<0, 16>::run([&]<int S>() { pp[S] = row_bcast<S>(ck) * yk; });
      }
#pragma unroll
      for (int i = K - 1; i >= 1; --i) {
        const float cp = cv[i - 1], yp = dyp[i - 1], dli = dl[i];
        Unroll<0, 16>::run(
            [&]<int S>() { pp[S] = __builtin_fmaf(fast_exp2(dli * A2[S]), pp[S], row_bcast<S>(cp) * yp); });
      }
      Unroll<0, 16>::run([&]<int S>() { mm[S] = fast_exp2(dl[0] * A2[S]) * pp[S]; });
    } else {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const float bi = bv[i];
        const float ui = u[i];
        Unroll<0, 16>::run([&]<int S>() {
          ab[i][S] = fast_exp2(dl[i] * A2[S]);
          bu[i][S] = row_bcast<S>(bi) * ui;
          bt[S] = (i == 0) ? bu[0][S] : __builtin_fmaf(ab[i][S], bt[S], bu[i][S]);
        });
      }
      // the reverse fold over the K = 2 steps: m = Abar_0 (c_0 + Abar_1 c_1)
      const float c0 = cv[0], c1 = cv[1], y0 = dyp[0], y1 = dyp[1];
      Unroll<0, 16>::run([&]<int S>() {
        cy[0][S] = row_bcast<S>(c0) * y0;
        cy[1][S] = row_bcast<S>(c1) * y1;
        // opaque from here: pass 2 reads the products, so the broadcasts are
        // not kept to form them again there
        asm volatile("" : "+v"(cy[0][S]), "+v"(cy[1][S]));
        mm[S] = ab[0][S] * __builtin_fmaf(ab[1][S], cy[1][S], cy[0][S]);
      });
    }
    {
      float* pb = agg_b + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
      float* pm = agg_m + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
#pragma unroll
      for (int s = 0; s < 16; s += 4) {
        if constexpr (!FOLD)
          *reinterpret_cast<float4*>(pb + s * 16) = make_float4(bt[s], bt[s + 1], bt[s + 2], bt[s + 3]);
        *reinterpret_cast<float4*>(pm + s * 16) = make_float4(mm[s], mm[s + 1], mm[s + 2], mm[s + 3]);
      }
      if (g == 0) agg_sd[c * SDS + j] = sd;
    }
    __syncthreads();

    // ---- walks: forward states into the sub-chunks, adjoints out of them ----
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      if (pair_valid(k)) {
        int cc, n;
        pair_of(k, cc, n);
        const float a2 = a2s[cc * NS + n];
        float* pbw = agg_b + ((n / 4) * 16 + cc) * 4 + (n % 4);
        float* pmw = agg_m + ((n / 4) * 16 + cc) * 4 + (n % 4);
        const float* psd = agg_sd + cc * SDS;
        float av[SUB];
#pragma unroll
        for (int u4 = 0; u4 < SUB; u4 += 4) {
          const float4 v = *reinterpret_cast<const float4*>(psd + u4);
          av[u4] = fast_exp2(a2 * v.x);
          av[u4 + 1] = fast_exp2(a2 * v.y);
          av[u4 + 2] = fast_exp2(a2 * v.z);
          av[u4 + 3] = fast_exp2(a2 * v.w);
        }
        if constexpr (FOLD) {
#pragma unroll
          for (int u4 = 0; u4 < SUB; u4 += 4) {
            const float4 v = *reinterpret_cast<const float4*>(psd + u4);
            part_sd[k] += (v.x + v.y) + (v.z + v.w);
          }
        } else {
          float h = kAhead ? h_in[k] : load_h_in(kt, k);  // the state entering the tile
#pragma unroll
          for (int jj = 0; jj < SUB; ++jj) {
            const float bb = pbw[jj * (N / 4) * 64];
            pbw[jj * (N / 4) * 64] = h;
            h = __builtin_fmaf(av[jj], h, bb);
          }
        }
        float mu = mu_carry[k];
#pragma unroll
        for (int jj = SUB - 1; jj >= 0; --jj) {
          const float m = pmw[jj * (N / 4) * 64];
          if constexpr (!FOLD) pmw[jj * (N / 4) * 64] = mu;
          mu = __builtin_fmaf(av[jj], mu, m);
        }
        mu_carry[k] = mu;
      }
    }
    __syncthreads();
    if constexpr (FOLD) continue;  // the barrier above also orders the walk before the next pass 1

    // ---- pass 2: rebuild h over the lane's steps, run the adjoint back ----
    float hp[16], mu[16];
    {
      const float* pb = agg_b + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
      const float* pm = agg_m + ((j * (N / 4) + 4 * g) * 16 + c) * 4;
#pragma unroll
      for (int s = 0; s < 16; s += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pb + s * 16);
        hp[s] = v.x;
        hp[s + 1] = v.y;
        hp[s + 2] = v.z;
        hp[s + 3] = v.w;
        const float4 m = *reinterpret_cast<const float4*>(pm + s * 16);
        mu[s] = m.x;
        mu[s + 1] = m.y;
        mu[s + 2] = m.z;
        mu[s + 3] = m.w;
      }
    }
    __syncthreads();  // every wave has read its records: the next tile's pass 1 may overwrite them

    float hm[16];  // state after step 0
#pragma unroll
    for (int s = 0; s < 16; ++s) hm[s] = __builtin_fmaf(ab[0][s], hp[s], bu[0][s]);

    // The per-(step, channel) results of step i from the sums over all states
    // (sgb = sum_n g B, sda = sum_n g h Abar A, ypre = C.h for the gate):
    // dx, ddelta_raw, dz, and the dD and dbias accumulators.  The step's
    // offset from t_tile is soff_step in the scalar offset plus whatever voff
    // adds to the lane's own row.
    auto step_out = [&](int i, float sgb, float sda, float ypre, uint32_t voff, int soff_step)
                        __attribute__((always_inline)) {
      const float xi = xv[i], yi = dyp[i];
      if constexpr (GATE) ypre += dskip * xi;
      const float ddt = __builtin_fmaf(xi, sgb, sda * kLn2);  // A = A2 ln 2
      const float ddraw = ddt * fac[i];
      const float dxv = __builtin_fmaf(dl[i], sgb, yi * dskip);
      const uint32_t sx = static_cast<uint32_t>((t_tile + soff_step) * xd_step);
      if ((full || i < left) && (G == 1 || (i % G) == g)) {
        Elem<IO>::store(rdx, voff, sx, dxv);
        Elem<IO>::store(rdd, voff, sx, ddraw);
        if constexpr (GATE) {
          const float sz = sg_z[i];
          Elem<IO>::store(rdz, voff, sx, dyv[i] * ypre * sz * __builtin_fmaf(zv[i], 1.0f - sz, 1.0f));
        }
        dD_acc = __builtin_fmaf(yi, xi, dD_acc);
        db_acc += ddraw;
      } else if (j * K + i < L - t_tile && (G == 1 || (i % G) == g)) {
        Elem<IO>::store(rdx, voff, sx, 0.0f);
        Elem<IO>::store(rdd, voff, sx, 0.0f);
        if constexpr (GATE) Elem<IO>::store(rdz, voff, sx, 0.0f);
      }
    };
    float sg_p[K], sda_p[K], yp_p[K];  // G > 1: this lane's partial sums of each step (its 16 states)
#pragma unroll
    for (int ii = 0; ii < K; ++ii) {
      const int i = K - 1 - ii;  // steps in reverse
      // the state after step i (hn) and the one before it (hb)
      float hn[16];
      if (i == 1) {
#pragma unroll
        for (int s = 0; s < 16; ++s) hn[s] = __builtin_fmaf(ab[1][s], hm[s], bu[1][s]);
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) hn[s] = hm[s];
      }
      const float(&hb)[16] = (i == 1) ? hm : hp;
      const float yi = dyp[i];
      // mu becomes the adjoint of the state after step i: mu + dyp * C
#pragma unroll
      for (int s = 0; s < 16; ++s) mu[s] += cy[i][s];
      float sg4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      dot16_row_bcast(sg4, bv[i], mu);  // sum_n g B
      float ypre = 0.0f;
      if constexpr (GATE) {
        float yp4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        dot16_row_bcast(yp4, cv[i], hn);
        ypre = (yp4[0] + yp4[1]) + (yp4[2] + yp4[3]);
      }
      float sda4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      float vb[16], vc[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        vb[s] = mu[s] * u[i];
        vc[s] = yi * hn[s];
        mu[s] = ab[i][s] * mu[s];  // the adjoint before step i
        const float daa = mu[s] * hb[s];
        sda4[s & 3] = __builtin_fmaf(daa, A2[s], sda4[s & 3]);
        dAl[s] = __builtin_fmaf(daa, dl[i], dAl[s]);
      }
      // dB, dC at this step: sums over the 16 channels of the row (lane c
      // gets state 16 g + c)
      const float sB = row_reduce_scatter16(vb, c);
      const float sC = row_reduce_scatter16(vc, c);
      if (full || i < left) {
        const int64_t t = t_tile + j * K + i;
        wdB[t * N + 16 * g + c] = sB;
        wdC[t * N + 16 * g + c] = sC;
      }
      sg_p[i] = (sg4[0] + sg4[1]) + (sg4[2] + sg4[3]);
      sda_p[i] = (sda4[0] + sda4[1]) + (sda4[2] + sda4[3]);
      yp_p[i] = ypre;
      if constexpr (G == 1) step_out(i, sg_p[i], sda_p[i], ypre, off_xd, i);
    }
    if constexpr (G > 1) {
      // Reduce-scatter of the two steps' partial sums over the state-group
      // rows, in the order (r0 + r1) + (r2 + r3): v_permlane16_swap of the
      // partials of steps 0 and 1 leaves row 2q (2q + 1) of each pair with
      // both rows' step 0 (1); at G = 4 v_permlane32_swap then adds the two
      // halves.  Row r ends with the totals of step r % 2, the step it
      // discretised and (rows g < 2 at G = 4) stores.
      auto scatter = [](float v0, float v1) __attribute__((always_inline)) {
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(v0), "+v"(v1));
        float t = v0 + v1;
        if constexpr (G == 4) {
          float lo, hi;
          rows_swap32(t, lo, hi);
          t = lo + hi;
        }
        return t;
      };
      const float sgb = scatter(sg_p[0], sg_p[1]);
      const float sda = scatter(sda_p[0], sda_p[1]);
      const float ypre = GATE ? scatter(yp_p[0], yp_p[1]) : 0.0f;
      step_out(r & 1, sgb, sda, ypre, off_xd_own, 0);
    }
  }

  if constexpr (FOLD) {
    // the part's adjoint fold from zero, and its delta sums per channel
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      if (pair_valid(k)) {
        int cc, n;
        pair_of(k, cc, n);
        p.ws_M[(part - 1) * sblock + state_block + pair_offset(k)] = mu_carry[k];
        if (n == 0) p.ws_S[(static_cast<int64_t>(part - 1) * p.nb + b) * nd + cg * 16 + cc] = part_sd[k];
      }
    }
    return;
  }

  // dA: each lane's 16 states summed over the lanes of its channel (the
  // sub-chunks j), staged [state][channel][j] through agg_b.
#pragma unroll
  for (int s = 0; s < 16; ++s) agg_b[((16 * g + s) * 16 + c) * SUB + j] = dAl[s];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    if (pair_valid(k)) {
      int cc, n;
      pair_of(k, cc, n);
      const float* pa = agg_b + (n * 16 + cc) * SUB;
      float s4 = 0.0f;
#pragma unroll
      for (int u4 = 0; u4 < SUB; u4 += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pa + u4);
        s4 += (v.x + v.y) + (v.z + v.w);
      }
      dA_acc[k] = s4;
    }
  }

  // ---- per-(b, d) and per-(b, d, n) results ----
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    if (pair_valid(k)) {
      int cc, n;
      pair_of(k, cc, n);
      const int64_t o = state_block + pair_offset(k);
      if (p.dh0 != nullptr && part == 0) p.dh0[o] = mu_carry[k];
      p.ws_dA[part * sblock + o] = dA_acc[k];
    }
  }
  red[0][tid] = dD_acc;
  red[1][tid] = db_acc;
  __syncthreads();
  if (tid < 16) {
    // lanes of channel tid: lane index (w, r, c = tid) over all waves and rows
    float s0 = 0.0f, s1 = 0.0f;
    for (int ww = 0; ww < W; ++ww)
      for (int rr = 0; rr < 4; ++rr) {
        s0 += red[0][ww * 64 + rr * 16 + tid];
        s1 += red[1][ww * 64 + rr * 16 + tid];
      }
    p.ws_dD[(static_cast<int64_t>(part) * p.nb + b) * nd + cg * 16 + tid] = s0;
    p.ws_db[(static_cast<int64_t>(part) * p.nb + b) * nd + cg * 16 + tid] = s1;
  }
}

// Sums the partials in a fixed order: dB, dC over channel groups (zero past
// each row's valid length), dA_log = A * sum over (part, row) of dA, dD and
// dbias over (part, row).
struct ReduceParams {
  const float* ws_dB;
  const float* ws_dC;
  const float* ws_dA;
  const float* ws_dD;
  const float* ws_db;
  const float* A_log;
  const int32_t* valid_len;
  float* dB;
  float* dC;
  float* dA_log;
  float* dD;
  float* dbias;
  int64_t L;
  int32_t nb, nd, N, n_cg;
  int32_t rows;  // n_parts * nb partial rows of dA, dD, dbias
};

__global__ __launch_bounds__(256) void ssm_bwd_reduce_kernel(ReduceParams p) {
  const int64_t n_bc = static_cast<int64_t>(p.nb) * p.L * p.N;
  const int64_t n_dn = static_cast<int64_t>(p.nd) * p.N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_bc + n_dn + p.nd;
       i += stride) {
    if (i < n_bc) {
      const int64_t b = i / (p.L * p.N), t = (i / p.N) % p.L;
      int64_t len = p.L;
      if (p.valid_len != nullptr) {
        const int64_t v = p.valid_len[b];
        len = v < 0 ? 0 : (v > p.L ? p.L : v);
      }
      float sb = 0.0f, sc = 0.0f;
      if (t < len) {
        // eight groups' loads in flight at once; the additions stay in group
        // order
        int g = 0;
        for (; g + 8 <= p.n_cg; g += 8) {
          float vb[8], vc[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            vb[k] = p.ws_dB[(g + k) * n_bc + i];
            vc[k] = p.ws_dC[(g + k) * n_bc + i];
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            sb += vb[k];
            sc += vc[k];
          }
        }
        for (; g < p.n_cg; ++g) {
          sb += p.ws_dB[g * n_bc + i];
          sc += p.ws_dC[g * n_bc + i];
        }
      }
      p.dB[i] = sb;
      p.dC[i] = sc;
    } else if (i < n_bc + n_dn) {
      const int64_t k = i - n_bc;
      float s = 0.0f;
      for (int b = 0; b < p.rows; ++b) s += p.ws_dA[b * n_dn + k];
      p.dA_log[k] = s * -expf(p.A_log[k]);
    } else {
      const int64_t dd = i - n_bc - n_dn;
      float s0 = 0.0f, s1 = 0.0f;
      for (int b = 0; b < p.rows; ++b) {
        s0 += p.ws_dD[b * p.nd + dd];
        s1 += p.ws_db[b * p.nd + dd];
      }
      if (p.dD != nullptr) p.dD[dd] = s0;
      if (p.dbias != nullptr) p.dbias[dd] = s1;
    }
  }
}

template <typename IO, int G, bool SP, bool CL, bool GATE>
hipError_t bwd_launch_flags(const BwdParams& prm, bool wide, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(prm.nb) * prm.n_cg;
  if (prm.n_parts > 1) {
    // the fold of parts 1 .. n_parts-1 first, on the same stream
    hipLaunchKernelGGL((ssm_bwd_kernel<IO, G, kBwdW, SP, CL, GATE, true>),
                       dim3(static_cast<unsigned>(groups * (prm.n_parts - 1))), dim3(64 * kBwdW), 0, stream, prm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ssm_bwd_kernel<IO, G, kBwdW, SP, CL, GATE, false>),
                       dim3(static_cast<unsigned>(groups * prm.n_parts)), dim3(64 * kBwdW), 0, stream, prm);
  } else if (wide) {
    hipLaunchKernelGGL((ssm_bwd_kernel<IO, G, 2 * kBwdW, SP, CL, GATE, false>), dim3(static_cast<unsigned>(groups)),
                       dim3(64 * 2 * kBwdW), 0, stream, prm);
  } else {
    hipLaunchKernelGGL((ssm_bwd_kernel<IO, G, kBwdW, SP, CL, GATE, false>), dim3(static_cast<unsigned>(groups)),
                       dim3(64 * kBwdW), 0, stream, prm);
  }
  return hipGetLastError();
}

template <typename IO, int G>
hipError_t bwd_launch(const BwdParams& prm, bool sp, bool wide, hipStream_t stream) {
  const bool gate = prm.z != nullptr;
  if (sp) {
    if (prm.clamp)
      return gate ? bwd_launch_flags<IO, G, true, true, true>(prm, wide, stream)
                  : bwd_launch_flags<IO, G, true, true, false>(prm, wide, stream);
    return gate ? bwd_launch_flags<IO, G, true, false, true>(prm, wide, stream)
                : bwd_launch_flags<IO, G, true, false, false>(prm, wide, stream);
  }
  if (prm.clamp)
    return gate ? bwd_launch_flags<IO, G, false, true, true>(prm, wide, stream)
                : bwd_launch_flags<IO, G, false, true, false>(prm, wide, stream);
  return gate ? bwd_launch_flags<IO, G, false, false, true>(prm, wide, stream)
              : bwd_launch_flags<IO, G, false, false, false>(prm, wide, stream);
}

template <typename IO>
hipError_t bwd_launch_io(int G, const BwdParams& prm, bool sp, bool wide, hipStream_t stream) {
  switch (G) {
    case 1:
      return bwd_launch<IO, 1>(prm, sp, wide, stream);
    case 2:
      return bwd_launch<IO, 2>(prm, sp, wide, stream);
    default:
      return bwd_launch<IO, 4>(prm, sp, wide, stream);
  }
}

constexpr int64_t kBwdMaxParts = 16;

// Workspace floats: dB and dC partials per channel group; dA, dD and dbias per
// (part, row); the fold's adjoint and delta sums per (part >= 1, row) -- sized
// for the largest split.
int64_t bwd_ws_floats(int64_t nb, int64_t L, int64_t nd, int64_t N) {
  return 2 * (nd / 16) * nb * L * N + kBwdMaxParts * (nb * nd * N + 2 * nb * nd) +
         (kBwdMaxParts - 1) * (nb * nd * N + nb * nd);
}

// dst[i] = src[i], or 0 with no src: the outputs of a call with no time
// steps.  A kernel rather than a runtime copy or memset, so that a captured
// call holds kernel nodes only.
__global__ void copy_or_zero_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : 0.0f;
}

}  // namespace

extern "C" {

int64_t ssm_scan_bwd_chunk_len(int64_t dstate) { return bwd_tile(dstate); }

int64_t ssm_scan_bwd_workspace_bytes(const ssm_scan_dims* dims) {
  if (dims == nullptr || dims->batch < 0 || dims->seqlen < 0 || dims->dim < 0) return -1;
  if (bwd_tile(dims->dstate) == 0 || dims->dim % 16 != 0) return -1;
  return 4 * bwd_ws_floats(dims->batch, dims->seqlen, dims->dim, dims->dstate);
}

// Checks run in this order: dims and flags; pointers; alignment; aliasing;
// the handle; the current device.  Nothing is enqueued unless all pass.
int ssm_selective_scan_bwd(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B,
                           const void* C, const float* D, const int32_t* valid_len, const ssm_scan_dims* dims,
                           const ssm_scan_fwd_extras* extras, const ssm_scan_bwd_io* io, void* stream) {
  if (dims == nullptr || io == nullptr) return SSM_ERR_INVALID_ARG;
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
  if (nb > 0 && nd > 0 && (nb * (nd / 16) > 0x7fffffffLL || nb > 0x7fffffffLL || nd > 0x7fffffffLL))
    return SSM_ERR_UNSUPPORTED;
  const int64_t esz = dims->io_dtype == SSM_IO_BF16 ? 2 : 4;
  if (L > 0 && L * (N > nd ? N : nd) * esz > 0x7fffffffLL) return SSM_ERR_UNSUPPORTED;
  const ssm_scan_fwd_extras none = {nullptr, nullptr, nullptr, nullptr, 0, 0, nullptr, 0};
  const ssm_scan_fwd_extras& ex = extras ? *extras : none;
  const int64_t T = bwd_tile(N);
  const int64_t n_tiles = L > 0 ? (L + T - 1) / T : 0;
  const int64_t need = 4 * bwd_ws_floats(nb, L, nd, N);
  if (io->workspace_bytes < need) return SSM_ERR_INVALID_ARG;

  const bool empty = (nb == 0 || nd == 0);
  const size_t e = static_cast<size_t>(esz);
  const size_t n_xd = static_cast<size_t>(nb) * L * nd, n_bc = static_cast<size_t>(nb) * L * N;
  const size_t n_state = static_cast<size_t>(nb) * nd * N;
  if (!empty) {
    if (A_log == nullptr || io->dA_log == nullptr || io->workspace == nullptr) return SSM_ERR_INVALID_ARG;
    if (L > 0 && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || io->dy == nullptr ||
                  io->dx == nullptr || io->ddelta == nullptr || io->dB == nullptr || io->dC == nullptr))
      return SSM_ERR_INVALID_ARG;
    if (L > 0 && n_tiles > 1 && io->chunk_states == nullptr) return SSM_ERR_INVALID_ARG;
    if (L > 0 && ex.z != nullptr && io->dz == nullptr) return SSM_ERR_INVALID_ARG;
    const void* es[] = {x, delta, B, C, ex.z, io->dy, io->dx, io->ddelta, io->dz};
    for (const void* q : es)
      if (!aligned(q, e)) return SSM_ERR_UNSUPPORTED;
    const void* fs[] = {A_log, D, valid_len, ex.h0, ex.delta_bias, io->dh_last, io->chunk_states, io->dA_log,
                        io->dB, io->dC, io->dD, io->ddelta_bias, io->dh0, io->workspace};
    for (const void* q : fs)
      if (!aligned(q, 4)) return SSM_ERR_UNSUPPORTED;
    const size_t bxd = L > 0 ? n_xd * e : 0;
    // chunk_states is read as [batch, n_tiles, dim, dstate] up to chunk
    // n_tiles - 2 of the last row
    const size_t bcs = n_tiles > 1 ? static_cast<size_t>(nb * n_tiles - 1) * nd * N * 4 : 0;
    const void* ins[] = {x, delta, B, C, A_log, D, valid_len, L > 0 ? ex.z : nullptr, ex.h0, ex.delta_bias,
                         L > 0 ? io->dy : nullptr, io->dh_last, io->chunk_states};
    const size_t ins_n[] = {n_xd * e, n_xd * e, n_bc * e, n_bc * e, static_cast<size_t>(nd) * N * 4,
                            D ? static_cast<size_t>(nd) * 4 : 0, valid_len ? static_cast<size_t>(nb) * 4 : 0,
                            ex.z ? n_xd * e : 0, ex.h0 ? n_state * 4 : 0, ex.delta_bias ? static_cast<size_t>(nd) * 4 : 0,
                            bxd, io->dh_last ? n_state * 4 : 0, io->chunk_states ? bcs : 0};
    void* outs[] = {io->dx, io->ddelta, io->dz, io->dA_log, io->dB, io->dC, io->dD, io->ddelta_bias, io->dh0,
                    io->workspace};
    const size_t outs_n[] = {bxd, bxd, ex.z ? bxd : 0, static_cast<size_t>(nd) * N * 4, L > 0 ? n_bc * 4 : 0,
                             L > 0 ? n_bc * 4 : 0, io->dD ? static_cast<size_t>(nd) * 4 : 0,
                             io->ddelta_bias ? static_cast<size_t>(nd) * 4 : 0, io->dh0 ? n_state * 4 : 0,
                             static_cast<size_t>(need)};
    for (int o = 0; o < 10; ++o) {
      for (int k = 0; k < 13; ++k)
        if (overlaps(outs[o], outs_n[o], ins[k], ins_n[k])) return SSM_ERR_ALIAS;
      for (int o2 = o + 1; o2 < 10; ++o2)
        if (overlaps(outs[o], outs_n[o], outs[o2], outs_n[o2])) return SSM_ERR_ALIAS;
    }
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
  float* ws = static_cast<float*>(io->workspace);
  const int64_t n_cg = nd / 16;
  BwdParams prm;
  prm.x = x;
  prm.delta = delta;
  prm.A_log = A_log;
  prm.B = B;
  prm.C = C;
  prm.D = D;
  prm.valid_len = valid_len;
  prm.h0 = ex.h0;
  prm.delta_bias = ex.delta_bias;
  prm.z = ex.z;
  prm.chunk_states = io->chunk_states;
  prm.dy = io->dy;
  prm.dh_last = io->dh_last;
  prm.dx = io->dx;
  prm.ddelta = io->ddelta;
  prm.dz = ex.z != nullptr ? io->dz : nullptr;
  prm.dh0 = io->dh0;
  // Time split: while the (row, channel group) grid would leave CUs idle (at
  // most two thirds as many groups as CUs), cut time into parts of whole
  // tiles: about two workgroups per resident slot, at most 16 parts and at
  // least four tiles per part.  Above that the split costs more than it
  // balances (measured at 4096 steps: 192 groups 3 / 6 / 8 % slower split at
  // dstate 16 / 32 / 64; dstate 16, 256 groups 0.369 ms split, 0.338 ms not;
  // 448 groups 0.678 / 0.570 ms).  With few groups the cap matters: 32 groups
  // of 16384 steps 0.258 ms in 8 parts, 0.190 ms in 16; at 128 groups 16
  // parts lost 1-4 % against the 8 this rule gives (except 2 % gained on
  // 32768 steps).
  const int64_t groups = nb * n_cg;
  const int64_t slots = 2 * static_cast<int64_t>(handle->cu_count);
  int64_t parts = 1, part_len = L;
  if (3 * groups <= 2 * static_cast<int64_t>(handle->cu_count)) {
    int64_t want = (2 * slots + groups - 1) / groups;
    if (want > kBwdMaxParts) want = kBwdMaxParts;
    if (want > n_tiles / 4) want = n_tiles / 4;
    if (want > 1) {
      const int64_t per = (n_tiles + want - 1) / want;
      parts = (n_tiles + per - 1) / per;
      part_len = per * T;
    }
  }
  prm.ws_dB = ws;
  prm.ws_dC = ws + n_cg * nb * L * N;
  prm.ws_dA = ws + 2 * n_cg * nb * L * N;
  prm.ws_dD = prm.ws_dA + kBwdMaxParts * nb * nd * N;
  prm.ws_db = prm.ws_dD + kBwdMaxParts * nb * nd;
  prm.ws_M = prm.ws_db + kBwdMaxParts * nb * nd;
  prm.ws_S = prm.ws_M + (kBwdMaxParts - 1) * nb * nd * N;
  prm.part_len = part_len;
  prm.n_parts = static_cast<int32_t>(parts);
  prm.L = L;
  prm.n_chunks = n_tiles;
  prm.nb = static_cast<int32_t>(nb);
  prm.nd = static_cast<int32_t>(nd);
  prm.n_cg = static_cast<int32_t>(n_cg);
  prm.clamp = dims->delta_clamp;
  // four-wave workgroups, two per CU, when unsplit and more than one per CU
  prm.pair_rows =
      use_length_pairing(valid_len, parts, nb, n_cg, handle->cu_count) && groups > handle->cu_count ? 1 : 0;
  prm.dmin = dims->delta_min;
  prm.dmax = dims->delta_max;
  const int G = static_cast<int>(N / 16);
  if (L == 0) {
    // No steps: the adjoint of the initial state is dh_last; every other
    // gradient is zero.
    float* outs[] = {io->dA_log, io->dD, io->ddelta_bias, io->dh0};
    const float* srcs[] = {nullptr, nullptr, nullptr, io->dh_last};
    const int64_t cnt[] = {nd * N, nd, nd, nb * nd * N};
    for (int k = 0; k < 4; ++k)
      if (outs[k] != nullptr)
        hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<unsigned>((cnt[k] + 255) / 256)), dim3(256), 0, s,
                           outs[k], srcs[k], cnt[k]);
    return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  // Eight-wave workgroups when an unsplit grid has at most one workgroup per
  // CU (four-wave ones would leave half of each CU's SIMD slots empty).
  const bool wide = parts == 1 && groups <= static_cast<int64_t>(handle->cu_count);
  hipError_t err = dims->io_dtype == SSM_IO_BF16
                       ? bwd_launch_io<uint16_t>(G, prm, dims->delta_softplus != 0, wide, s)
                       : bwd_launch_io<float>(G, prm, dims->delta_softplus != 0, wide, s);
  if (err != hipSuccess) return SSM_ERR_HIP;
  ReduceParams rp;
  rp.ws_dB = prm.ws_dB;
  rp.ws_dC = prm.ws_dC;
  rp.ws_dA = prm.ws_dA;
  rp.ws_dD = prm.ws_dD;
  rp.ws_db = prm.ws_db;
  rp.A_log = A_log;
  rp.valid_len = valid_len;
  rp.dB = io->dB;
  rp.dC = io->dC;
  rp.dA_log = io->dA_log;
  rp.dD = io->dD;
  rp.dbias = io->ddelta_bias;
  rp.L = L;
  rp.nb = static_cast<int32_t>(nb);
  rp.nd = static_cast<int32_t>(nd);
  rp.N = static_cast<int32_t>(N);
  rp.n_cg = static_cast<int32_t>(n_cg);
  rp.rows = static_cast<int32_t>(parts * nb);
  const int64_t work = nb * L * N + nd * N + nd;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ssm_bwd_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, rp);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
