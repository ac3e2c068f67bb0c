// Current-scaling FP8 casts (Megatron-LM tuning post, mixed-precision
// section: E4M3 / E5M2 operands for the matrix products, the scale of a
// tensor taken from the tensor itself).
//
//   amax:  max |x| over a logical bf16 matrix (one or two segments), one
//          vector atomic max per workgroup on the float's bits (non-negative
//          floats order like their bit patterns).
//   cast:  code = RNE(clamp(x * s, -FMAX, FMAX)) with s = FMAX / amax, x * s
//          one fp32 multiply; written row-wise (same layout) and/or
//          transposed, so that every FP8 product reads two k-contiguous
//          operands.  64 x 64 tiles: each thread loads a 4 x 4 block (four
//          8-byte loads), the transpose goes through LDS as 4-byte columns
//          of codes and leaves as 16-byte rows.  Padding (up to the output's
//          leading dimension) is written as zero codes, so that products
//          can run K up to a whole number of 128-wide k-steps.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int CT = 64;      // cast tile (rows and columns of X)
constexpr int TS = CT + 4;  // LDS row stride in bytes of the transposed tile

__device__ __forceinline__ const u16* src_at(const CastSrc& x, int r, int c) {
  if (x.split_on_rows)
    return r < x.split ? x.p0 + static_cast<size_t>(r) * x.ld0 + c
                       : x.p1 + static_cast<size_t>(r - x.split) * x.ld1 + c;
  return c < x.split ? x.p0 + static_cast<size_t>(r) * x.ld0 + c
                     : x.p1 + static_cast<size_t>(r) * x.ld1 + (c - x.split);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__global__ __launch_bounds__(256) void amax_kernel(CastSrc x, float* amax) {
  __shared__ uint32_t part[4];
  const uint32_t cpr = static_cast<uint32_t>(x.C) / 8;  // 16-byte chunks per row
  const uint32_t total = static_cast<uint32_t>(x.R) * cpr;
  uint32_t m = 0;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
    const int r = static_cast<int>(i / cpr), c = static_cast<int>(i % cpr) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(src_at(x, r, c));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = umax(m, (w[k] & 0x7fffu) << 16);
      m = umax(m, w[k] & 0x7fff0000u);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = umax(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = umax(umax(part[0], part[1]), umax(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), m);
  }
}

// Four codes (x0..x3 scaled and clamped) packed low byte first.
template <int FMT>
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, float s) {
  constexpr float M = fp8_max(FMT);
  const float y0 = fminf(fmaxf(x0 * s, -M), M), y1 = fminf(fmaxf(x1 * s, -M), M);
  const float y2 = fminf(fmaxf(x2 * s, -M), M), y3 = fminf(fmaxf(x3 * s, -M), M);
  int w;
  if constexpr (FMT == FP8_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(y2, y3, w, true);
  }
  return static_cast<uint32_t>(w);
}

// One 64 x 64 tile of X at (r0, c0).  Thread (br, bc) = (tid / 16, tid % 16)
// owns rows r0 + 4 br .. +3 and columns c0 + 4 bc .. +3.
template <int FMT>
__global__ __launch_bounds__(256) void cast_kernel(CastSrc x, const float* amax, uint8_t* rows,
                                                   int ldr, uint8_t* cols, int ldc) {
  __shared__ uint32_t tt[CT * TS / 4];
  const float s = fp8_scale(*amax, fp8_max(FMT));
  const int r0 = blockIdx.y * CT, c0 = blockIdx.x * CT;
  const int tid = threadIdx.x, br = tid >> 4, bc = tid & 15;
  const int c = c0 + 4 * bc;
  uint32_t q[4];  // q[i]: codes of row r0 + 4 br + i, columns c .. c+3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 4 * br + i;
    uint2 v = make_uint2(0u, 0u);
    if (r < x.R && c < x.C) v = *reinterpret_cast<const uint2*>(src_at(x, r, c));
    q[i] = quant4<FMT>(lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y), s);
  }
  if (rows != nullptr && c0 < ldr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 4 * br + i;
      if (r < x.R) *reinterpret_cast<uint32_t*>(rows + static_cast<size_t>(r) * ldr + c) = q[i];
    }
  }
  if (cols == nullptr || r0 >= ldc) return;
  // column j of the 4 x 4 block: rows 4 br .. +3 as one 4-byte word
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = ((q[0] >> (8 * j)) & 0xffu) | (((q[1] >> (8 * j)) & 0xffu) << 8) |
                       (((q[2] >> (8 * j)) & 0xffu) << 16) | (((q[3] >> (8 * j)) & 0xffu) << 24);
    tt[((4 * bc + j) * TS + 4 * br) / 4] = w;
  }
  __syncthreads();
  // output row oc = column c0 + oc of X, bytes 16 (tid % 4) .. +15
  const int oc = tid >> 2, ob = (tid & 3) * 16;
  if (c0 + oc >= x.C) return;
  uint4 o;
  o.x = tt[(oc * TS + ob) / 4];
  o.y = tt[(oc * TS + ob + 4) / 4];
  o.z = tt[(oc * TS + ob + 8) / 4];
  o.w = tt[(oc * TS + ob + 12) / 4];
  *reinterpret_cast<uint4*>(cols + static_cast<size_t>(c0 + oc) * ldc + r0 + ob) = o;
}

bool src_ok(const CastSrc& x) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  return x.p0 != nullptr && x.p1 != nullptr && al(x.p0) && al(x.p1) && x.R > 0 && x.C > 0 &&
         x.C % 8 == 0 && x.ld0 % 8 == 0 && x.ld1 % 8 == 0 && x.split % 8 == 0 && x.split > 0;
}

}  // namespace

hipError_t launch_amax(const CastSrc& x, float* amax, hipStream_t s) {
  if (!src_ok(x) || amax == nullptr) return hipErrorInvalidValue;
  const long chunks = static_cast<long>(x.R) * (x.C / 8);
  if (chunks >= (1L << 31)) return hipErrorInvalidValue;
  const int blocks = static_cast<int>(std::min<long>((chunks + 255) / 256, 1024));
  hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(256), 0, s, x, amax);
  return hipGetLastError();
}

hipError_t launch_cast_fp8(const CastSrc& x, Fp8Format fmt, const float* amax, uint8_t* rows,
                           int ldr, uint8_t* cols, int ldc, hipStream_t s) {
  if (!src_ok(x) || amax == nullptr || (rows == nullptr && cols == nullptr))
    return hipErrorInvalidValue;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (rows != nullptr && (ldr < x.C || ldr % CT != 0 || !al(rows))) return hipErrorInvalidValue;
  if (cols != nullptr && (ldc < x.R || ldc % CT != 0 || !al(cols))) return hipErrorInvalidValue;
  const int rspan = cols != nullptr ? std::max(x.R, ldc) : x.R;
  const int cspan = rows != nullptr ? std::max(x.C, ldr) : x.C;
  const dim3 grid((cspan + CT - 1) / CT, (rspan + CT - 1) / CT);
  if (fmt == FP8_E4M3)
    hipLaunchKernelGGL(cast_kernel<FP8_E4M3>, grid, dim3(256), 0, s, x, amax, rows, ldr, cols, ldc);
  else
    hipLaunchKernelGGL(cast_kernel<FP8_E5M2>, grid, dim3(256), 0, s, x, amax, rows, ldr, cols, ldc);
  return hipGetLastError();
}

}  // namespace ptb
