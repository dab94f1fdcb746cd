// Internals shared by the forward and backward sources of the HIP library:
// the handle, buffer-resource element access, and the device math helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

struct ssm_scan_handle_s {
  int device;
  int cu_count;
  float* scratch;  // this device's copy of the forward's static scratch array
};

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element access ------------------------------------------------------
//
// Every tensor row a workgroup touches is addressed through a buffer resource
// (base in SGPRs) with a fixed per-lane byte offset in a VGPR and the per-step
// offset in an SGPR, so the hot loop does no per-lane address arithmetic.  The
// host guarantees that a row spans fewer than 2^31 bytes.

using rsrc_t = __amdgpu_buffer_rsrc_t;

// Word 3 of a gfx9 buffer resource: 32-bit data format, everything else zero.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy bits of buffer instructions.  Everything uses the default
// policy: a workgroup touches 32-byte pieces of the 128-byte lines of x,
// delta, y (16 channels of bf16), and with the non-temporal hint those pieces
// went to HBM separately (1.36x the algorithmic bytes at the headline shape);
// cached, the neighbouring workgroups' pieces merge in L2 (1.05x).
constexpr int kCached = 0;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

template <typename IO>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  template <int AUX>
  static __device__ __forceinline__ float load(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, kCached);
  }
};

// bf16 is carried as its 16-bit pattern; widening to fp32 is exact.
template <>
struct Elem<uint16_t> {
  static constexpr int kBytes = 2;
  template <int AUX>
  static __device__ __forceinline__ float load(rsrc_t r, uint32_t voff, uint32_t soff) {
    const uint32_t u = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX);
    return __builtin_bit_cast(float, u << 16);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    // v_cvt_pk_bf16_f32: round to nearest even.
    const __bf16 h = static_cast<__bf16>(v);
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), r, voff, soff, kCached);
  }
};

// ---- math ----------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// softplus(v) = max(v, 0) + log1p(e) with e = exp(-|v|) in (0, 1].  With
// w = fl(1 + e), the rounding error d = (1 + e) - w = e - (w - 1) is computed
// exactly (Dekker's Fast2Sum, "A floating-point technique for extending the
// available precision", 1971: 1 >= e, and w - 1 is exact for w in [1, 2]), and
// log1p(e) = log(w) + log(1 + d/w) = log(w) + d/w to first order.  d stands in
// for d/w: they differ by d e / (1 + e), at most 2^-24 log1p(e).  When w
// rounds to 1, log(w) = 0 and the result is e.
__device__ __forceinline__ float log1p_of_exp_term(float e, float w) {
  const float d = e - (w - 1.0f);
  return __builtin_fmaf(__builtin_amdgcn_logf(w), kLn2, d);  // v_log_f32 is log2
}

__device__ __forceinline__ float softplus_f32(float v) {
  const float e = fast_exp2(-__builtin_fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  return __builtin_fmaxf(v, 0.0f) + log1p_of_exp_term(e, w);
}

// DPP row_newbcast:S -- every lane of a 16-lane row reads lane S of that row.
template <int S>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + S, 0xf, 0xf, true));
}

// y_m += C[s] * h[s] for s % 4 == m over the 16 states (four accumulators, so
// that consecutive instructions do not depend on each other), C[s] taken from
// lane s of the row by DPP row_newbcast fused into v_fmac_f32 (the compiler
// does not fuse a DPP move into v_fmac, so this is written out).  The leading
// s_nop covers the DPP hazards (a VALU write of the DPP source needs 2 wait
// states before the read, a VALU write of EXEC needs 5); c is not written
// inside the block.
__device__ __forceinline__ void dot16_row_bcast(float (&y)[4], float c, const float (&h)[16]) {
  asm volatile(
      "s_nop 4\n\t"
      "v_fmac_f32_dpp %0, %4, %5 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %6 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %7 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %8 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %9 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %10 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %11 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %12 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %13 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %14 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %15 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %16 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %4, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %4, %18 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %4, %19 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %4, %20 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3])
      : "v"(c), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]), "v"(h[6]), "v"(h[7]),
        "v"(h[8]), "v"(h[9]), "v"(h[10]), "v"(h[11]), "v"(h[12]), "v"(h[13]), "v"(h[14]), "v"(h[15]));
}

// Row exchanges between the four 16-lane rows of a wave.  With both operands
// v, v_permlane16_swap leaves the rows [0, 0, 2, 2] of v in the first operand
// and [1, 1, 3, 3] in the second; v_permlane32_swap leaves [0, 1, 0, 1] and
// [2, 3, 2, 3].  s_nop 1 covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void rows_swap16(float v, float& lo, float& hi) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}
__device__ __forceinline__ void rows_swap32(float v, float& lo, float& hi) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}

// Length-paired rows.  A grid of exactly two (row, channel-group) workgroups
// per CU, dealt to the 8 XCDs round-robin (XCD = bid % 8, bid / 8 the order
// within it): the first half of an XCD's workgroups takes one slot of each of
// its CUs, the second half the other, in the same CU order.  With rows of
// different lengths, the longer rows go to the first slots in length order
// and the shorter ones, in reverse, to the second, so that each CU holds one
// long and one short row; each XCD half still holds whole rows when the
// channel groups per row divide the CUs per XCD.  The rows (at most 64) are
// ranked in LDS by every workgroup: longest first, ties by index.  Called by
// every thread of the workgroup (it contains barriers).
__device__ __forceinline__ void length_paired_row(int64_t bid, int64_t groups, int n_cg, int nb, int64_t L,
                                                  const int32_t* valid_len, int32_t* row_lens, int32_t* row_order,
                                                  int& b, int& cg) {
  const int half = static_cast<int>(groups / 16);  // CUs per XCD
  const int x = static_cast<int>(bid % 8), m = static_cast<int>(bid / 8);
  const int pos = x * half + (m < half ? m : m - half);
  const int rank = m < half ? pos : static_cast<int>(groups) - 1 - pos;
  cg = rank % n_cg;
  const int tid = threadIdx.x;
  if (tid < nb) {
    const int64_t v = valid_len[tid];
    row_lens[tid] = static_cast<int32_t>(v < 0 ? 0 : (v > L ? L : v));
  }
  __syncthreads();
  if (tid < nb) {
    const int32_t lr = row_lens[tid];
    int above = 0;
    for (int o = 0; o < nb; ++o) above += (row_lens[o] > lr || (row_lens[o] == lr && o < tid)) ? 1 : 0;
    row_order[above] = tid;
  }
  __syncthreads();
  b = row_order[rank / n_cg];
}

// Whether a grid takes length-paired rows: rows with their own lengths, no
// time split, exactly two workgroups per CU, whole rows per XCD half, at most
// 64 rows.
inline bool use_length_pairing(const void* valid_len, int64_t parts, int64_t nb, int64_t n_cg, int64_t cus) {
  const int64_t groups = nb * n_cg;
  return valid_len != nullptr && parts == 1 && nb <= 64 && n_cg > 0 && cus % 8 == 0 && groups == 2 * cus &&
         (cus / 8) % n_cg == 0;
}

template <int S, int K>
struct Unroll {
  template <typename F>
  static __device__ __forceinline__ void run(F&& f) {
    f.template operator()<S>();
    Unroll<S + 1, K>::run(f);
  }
};
template <int K>
struct Unroll<K, K> {
  template <typename F>
  static __device__ __forceinline__ void run(F&&) {}
};

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

inline bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace
