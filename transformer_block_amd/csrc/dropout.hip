// Dropout kernels for gfx950 (MegaScale reading notes, section 1.3: dropout
// fused into the layer, its activations kept for backward).  The mask is
// never stored: every bit is Philox-4x32-10 of (seed, stream, element), so
// the backward regenerates exactly the mask the forward's [O ; FC2] epilogue
// applied (the "kept" activation is the key that reproduces it).  Both
// kernels are HBM-bound elementwise passes: 8 elements (two generator calls)
// per thread per iteration, 16-byte accesses.
#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int DROP_THREADS = 256;

__global__ __launch_bounds__(DROP_THREADS) void dropout_apply_kernel(const u16* __restrict__ src,
                                                                     u16* __restrict__ dst,
                                                                     uint32_t n8, Dropout d) {
  for (uint32_t i = blockIdx.x * DROP_THREADS + threadIdx.x; i < n8;
       i += gridDim.x * DROP_THREADS) {
    const uint4 in = reinterpret_cast<const uint4*>(src)[i];
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[2 * j] = lo_bf(w[j]); v[2 * j + 1] = hi_bf(w[j]); }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 r = philox4x32_10(make_uint4(2 * i + q, d.stream, 0u, 0u), d.k0, d.k1);
      v[4 * q + 0] = r.x >= d.t ? v[4 * q + 0] * d.scale : 0.0f;
      v[4 * q + 1] = r.y >= d.t ? v[4 * q + 1] * d.scale : 0.0f;
      v[4 * q + 2] = r.z >= d.t ? v[4 * q + 2] * d.scale : 0.0f;
      v[4 * q + 3] = r.w >= d.t ? v[4 * q + 3] * d.scale : 0.0f;
    }
    reinterpret_cast<uint4*>(dst)[i] =
        make_uint4(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]), pack2bf(v[4], v[5]),
                   pack2bf(v[6], v[7]));
  }
}

__global__ __launch_bounds__(DROP_THREADS) void dropout_mask_kernel(uint8_t* __restrict__ mask,
                                                                    uint32_t groups, uint32_t n,
                                                                    Dropout d) {
  for (uint32_t j = blockIdx.x * DROP_THREADS + threadIdx.x; j < groups;
       j += gridDim.x * DROP_THREADS) {
    const uint4 r = philox4x32_10(make_uint4(j, d.stream, 0u, 0u), d.k0, d.k1);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * j + q < n) mask[4 * j + q] = w[q] >= d.t ? 1 : 0;
  }
}

int grid_for(long items) {
  const long g = (items + DROP_THREADS - 1) / DROP_THREADS;
  return static_cast<int>(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

}  // namespace

hipError_t launch_dropout_apply(const u16* src, u16* dst, long n, const Dropout& d,
                                hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 8 != 0 || n >= (1L << 32)) return hipErrorInvalidValue;
  const long n8 = n / 8;
  hipLaunchKernelGGL(dropout_apply_kernel, dim3(grid_for(n8)), dim3(DROP_THREADS), 0, s, src, dst,
                     static_cast<uint32_t>(n8), d);
  return hipGetLastError();
}

hipError_t launch_dropout_mask(uint8_t* mask, long n, const Dropout& d, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n >= (1L << 32) - 4) return hipErrorInvalidValue;
  const long groups = (n + 3) / 4;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3(grid_for(groups)), dim3(DROP_THREADS), 0, s, mask,
                     static_cast<uint32_t>(groups), static_cast<uint32_t>(n), d);
  return hipGetLastError();
}

}  // namespace ptb
