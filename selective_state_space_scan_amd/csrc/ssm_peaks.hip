// Peak-rate microbenchmarks of the GPU the scan runs on, for the measured
// side of the roofline: HBM read and copy bandwidth, the plain fp32 FMA rate
// and the v_exp_f32 rate.  A separate library (libssmpeaks.so) that only the
// benchmark loads; the scan library does not depend on it.
//
// Every kernel is a bounded grid-stride or fixed-count loop over buffers the
// caller sizes; results are written so that the compiler keeps the work.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

// Sum of n4 float4 (HBM read): one partial per thread into out[grid threads].
__global__ __launch_bounds__(256) void peak_read(const float4* __restrict__ a, int64_t n4, float* __restrict__ out) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int64_t i = tid; i < n4; i += stride) {
    const float4 v = a[i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  out[tid] = (acc.x + acc.y) + (acc.z + acc.w);
}

// b = a over n4 float4 (HBM read + write).
__global__ __launch_bounds__(256) void peak_copy(const float4* __restrict__ a, float4* __restrict__ b, int64_t n4) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = tid; i < n4; i += stride) b[i] = a[i];
}

// iters x 16 independent FMAs per thread in the two-operand VOP2 form
// v_fmac_f32 with both multiplicands in VGPRs (acc += x * y; the VOP3 form and
// scalar operands issue more slowly), bounded: acc grows by x * y per step.
__global__ __launch_bounds__(256) void peak_fma(float* __restrict__ out, int iters, float s, float t) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const float x = s * static_cast<float>((tid & 7) + 1), y = t * static_cast<float>((tid & 3) + 1);
  float a[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] = 0.001f * static_cast<float>(tid + k);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) a[k] = __builtin_fmaf(x, y, a[k]);
  }
  float r = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) r += a[k];
  out[tid] = r;
}

// iters x 8 independent v_exp_f32 per thread (bounded: a <- 2^-a stays in (0, 1]).
__global__ __launch_bounds__(256) void peak_exp(float* __restrict__ out, int iters) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  float a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = 0.001f * static_cast<float>(tid + k);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = __builtin_amdgcn_exp2f(-a[k]);
  }
  out[tid] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// LDS access patterns for reading the LDS counters (SQ_INSTS_LDS,
// SQ_LDS_BANK_CONFLICT): iters accesses per wave of one pattern, each wave in
// a window of its own, addresses rotated every iteration so that nothing is
// loop-invariant.  In 32-bit words, lane l of a wave at iteration i:
//   0 ds_read_b32   word (l + i) % 64              (64 lanes, 64 banks: no conflict)
//   1 ds_write_b32  word (l + i) % 64
//   2 ds_read_b64   words 2 ((l + i) % 64) + {0, 1}
//   3 ds_read_b128  words 4 ((l + i) % 64) + {0..3} (consecutive quads)
//   4 ds_write_b128 words 4 ((l + i) % 64) + {0..3}
//   5 ds_read_b32   word i % 64 for every lane     (broadcast)
//   6 ds_read_b32   word 2 ((l + i) % 64)          (stride 2: two lanes per bank)
//   7 ds_read_b128  words 80 (l / 16) + 4 (i % 4) + {0..3}: the 16 lanes of a
//                   row read one quad, the four rows 80 words apart (the
//                   forward's readout of C staged in LDS)
//   8 two reads     words (l + i) % 64 and that + 256 (one ds_read2st64_b32:
//                   both addresses of a lane in the same bank, as in the
//                   forward's carry walk over consecutive record slots)
//   9 two reads     words (l + i) % 64 and that + 68 (one ds_read2_b32, the
//                   two addresses in different banks)
//  10 two writes    words (l + i) % 64 and that + 256 (one ds_write2st64_b32)
__global__ __launch_bounds__(256) void peak_lds(float* __restrict__ out, int iters, int pattern) {
  __shared__ __attribute__((aligned(16))) float buf[4 * 320];
  const int lane = threadIdx.x & 63;
  float* const win = buf + (threadIdx.x >> 6) * 320;
  for (int k = lane; k < 320; k += 64) win[k] = 0.001f * static_cast<float>(k);
  __syncthreads();
  float acc = 0.0f;
  for (int it = 0; it < iters; ++it) {
    const int r = (lane + it) & 63;
    switch (pattern) {
      case 0:
        acc += win[r];
        break;
      case 1:
        win[r] = acc + static_cast<float>(it);
        break;
      case 2: {
        const float2 v = *reinterpret_cast<const float2*>(win + 2 * r);
        acc += v.x + v.y;
        break;
      }
      case 3: {
        const float4 v = *reinterpret_cast<const float4*>(win + 4 * r);
        acc += (v.x + v.y) + (v.z + v.w);
        break;
      }
      case 4:
        *reinterpret_cast<float4*>(win + 4 * r) = make_float4(acc, acc + 1.0f, acc + 2.0f, static_cast<float>(it));
        break;
      case 5:
        acc += win[it & 63];
        break;
      case 6:
        acc += win[2 * r];
        break;
      case 7: {
        const float4 v = *reinterpret_cast<const float4*>(win + 80 * (lane >> 4) + 4 * (it & 3));
        acc += (v.x + v.y) + (v.z + v.w);
        break;
      }
      case 8:
        acc += win[r] * win[r + 256];
        break;
      case 9:
        acc += win[r] * win[r + 68];
        break;
      default:
        win[r] = acc;
        win[r + 256] = acc + 1.0f;
        break;
    }
  }
  __syncthreads();
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc + win[lane];
}

}  // namespace

extern "C" {

// Launch one microbenchmark on `stream` (a hipStream_t) and return 0, or -1
// for bad arguments, -4 for a launch error.  which: 0 read (a: n4 float4
// in, out: blocks*256 floats), 1 copy (a -> b, n4 float4 each), 2 fma
// (iters iterations of 16 FMAs per thread), 3 exp (iters iterations of 8
// exps per thread) and 4 LDS access pattern n4 (0..10, see peak_lds; iters
// accesses per wave), out: blocks*256 floats.  blocks: the grid size in
// 256-thread workgroups.
int ssm_peak_launch(int which, const void* a, void* b, int64_t n4, float* out, int blocks, int iters,
                    void* stream) {
  if (blocks <= 0 || iters < 0 || n4 < 0) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (which) {
    case 0:
      if (a == nullptr || out == nullptr) return -1;
      hipLaunchKernelGGL(peak_read, dim3(blocks), dim3(256), 0, s, static_cast<const float4*>(a), n4, out);
      break;
    case 1:
      if (a == nullptr || b == nullptr) return -1;
      hipLaunchKernelGGL(peak_copy, dim3(blocks), dim3(256), 0, s, static_cast<const float4*>(a),
                         static_cast<float4*>(b), n4);
      break;
    case 2:
      if (out == nullptr) return -1;
      hipLaunchKernelGGL(peak_fma, dim3(blocks), dim3(256), 0, s, out, iters, 1.0e-7f, 0.5f);
      break;
    case 3:
      if (out == nullptr) return -1;
      hipLaunchKernelGGL(peak_exp, dim3(blocks), dim3(256), 0, s, out, iters);
      break;
    case 4:
      if (out == nullptr || n4 > 10) return -1;
      hipLaunchKernelGGL(peak_lds, dim3(blocks), dim3(256), 0, s, out, iters, static_cast<int>(n4));
      break;
    default:
      return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
