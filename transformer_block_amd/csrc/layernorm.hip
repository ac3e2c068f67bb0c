// LayerNorm forward and backward for gfx950, HBM-bandwidth bound.
//
// The Parallel Transformer Block feeds one LayerNorm output to both the
// attention and the MLP branch (MegaScale reading notes, section 1.1, eq (4));
// norms are kept in higher precision (Megatron tuning post, mixed-precision
// section): statistics and reductions are fp32 here.
//
// Forward: one 256-thread workgroup per token row; the row (h <= 16384 bf16)
// is read once into registers with 16-byte loads, mean and variance come from
// two block reductions over the register copy, and a = gamma*(x-mu)*rstd+beta
// is written back in bf16 with 16-byte stores, together with its rounding
// residual a_lo = bf16(a_fp32 - a) (used where bf16 rounding of a would be
// amplified: the query/key projection feeding the softmax logits).
// Backward: each workgroup walks a strided set of rows, computes
//   dx = dy + rstd * (g - mean(g) - xhat * mean(g * xhat)),  g = da * gamma,
// and keeps per-column partial sums of dgamma = sum da*xhat and dbeta = sum da
// in registers; a second kernel reduces the per-workgroup partials.
#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int LN_THREADS = 256;
constexpr int LN_MAXCH = 8;  // 16-byte chunks per thread: h <= 8 * 8 * 256 = 16384
constexpr int LN_BWD_BLOCKS = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = lo_bf(w[i]); f[2 * i + 1] = hi_bf(w[i]); }
}

__global__ __launch_bounds__(LN_THREADS) void ln_fwd_kernel(const u16* __restrict__ x,
                                                            const u16* __restrict__ gamma,
                                                            const u16* __restrict__ beta,
                                                            u16* __restrict__ a,
                                                            u16* __restrict__ a_lo,
                                                            float* __restrict__ mu_out,
                                                            float* __restrict__ rstd_out,
                                                            int h, float eps) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int nch = h >> 3;
  const u16* xr = x + static_cast<size_t>(row) * h;
  float v[LN_MAXCH][8];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < LN_MAXCH; ++i) {
    const int c = tid + i * LN_THREADS;
    if (c < nch) {
      unpack8(*reinterpret_cast<const uint4*>(xr + c * 8), v[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += v[i][j];
    }
  }
  const float mu = block_sum(sum, red) / static_cast<float>(h);
  float sq = 0.0f;
#pragma unroll
  for (int i = 0; i < LN_MAXCH; ++i) {
    const int c = tid + i * LN_THREADS;
    if (c < nch) {
#pragma unroll
      for (int j = 0; j < 8; ++j) { const float t = v[i][j] - mu; sq += t * t; }
    }
  }
  const float var = block_sum(sq, red) / static_cast<float>(h);
  const float rstd = 1.0f / sqrtf(var + eps);
  u16* ar = a + static_cast<size_t>(row) * h;
  u16* alr = a_lo + static_cast<size_t>(row) * h;
#pragma unroll
  for (int i = 0; i < LN_MAXCH; ++i) {
    const int c = tid + i * LN_THREADS;
    if (c < nch) {
      float gm[8], bt[8];
      unpack8(*reinterpret_cast<const uint4*>(gamma + c * 8), gm);
      unpack8(*reinterpret_cast<const uint4*>(beta + c * 8), bt);
      uint32_t o[4], ol[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = (v[i][2 * j] - mu) * rstd * gm[2 * j] + bt[2 * j];
        const float v1 = (v[i][2 * j + 1] - mu) * rstd * gm[2 * j + 1] + bt[2 * j + 1];
        o[j] = pack2bf(v0, v1);
        ol[j] = pack2bf(v0 - lo_bf(o[j]), v1 - hi_bf(o[j]));
      }
      *reinterpret_cast<uint4*>(ar + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(alr + c * 8) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
    }
  }
  if (tid == 0) { mu_out[row] = mu; rstd_out[row] = rstd; }
}

constexpr int LNB_THREADS = 1024;
constexpr int LNB_WAVES = LNB_THREADS / 64;

// Two block-wide sums at once (one pair of barriers).
__device__ __forceinline__ float2 block_sum2(float a, float b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) { red[wave] = a; red[LNB_WAVES + wave] = b; }
  __syncthreads();
  float sa = 0.0f, sb = 0.0f;
#pragma unroll
  for (int w = 0; w < LNB_WAVES; ++w) { sa += red[w]; sb += red[LNB_WAVES + w]; }
  return make_float2(sa, sb);
}

__device__ __forceinline__ void load8f(const float* p, float* f) {
  const float4 d0 = *reinterpret_cast<const float4*>(p);
  const float4 d1 = *reinterpret_cast<const float4*>(p + 4);
  f[0] = d0.x; f[1] = d0.y; f[2] = d0.z; f[3] = d0.w;
  f[4] = d1.x; f[5] = d1.y; f[6] = d1.z; f[7] = d1.w;
}

// NCH = 16-byte chunks of a row per thread (h <= NCH * 8 * 1024).  The row is
// read twice: once for the two row sums and the column partials, once more
// (from cache) for dx, which keeps register use low enough for 16 waves/CU.
template <int NCH>
__global__ __launch_bounds__(LNB_THREADS) void ln_bwd_kernel(
    const float* __restrict__ da, const u16* __restrict__ x, const u16* __restrict__ gamma,
    const float* __restrict__ mu, const float* __restrict__ rstd, const u16* __restrict__ dy,
    u16* __restrict__ dx, float* __restrict__ partials, int T, int h) {
  __shared__ float red[2 * LNB_WAVES];
  const int tid = threadIdx.x;
  const int nch = h >> 3;
  const float inv_h = 1.0f / static_cast<float>(h);
  float gm[NCH][8], pg[NCH][8], pb[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * LNB_THREADS;
#pragma unroll
    for (int j = 0; j < 8; ++j) { pg[i][j] = 0.0f; pb[i][j] = 0.0f; gm[i][j] = 0.0f; }
    if (c < nch) unpack8(*reinterpret_cast<const uint4*>(gamma + c * 8), gm[i]);
  }
  for (int row = blockIdx.x; row < T; row += gridDim.x) {
    const float m = mu[row], r = rstd[row];
    const float* dar = da + static_cast<size_t>(row) * h;
    const u16* xr = x + static_cast<size_t>(row) * h;
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * LNB_THREADS;
      if (c < nch) {
        float xv[8], dv[8];
        unpack8(*reinterpret_cast<const uint4*>(xr + c * 8), xv);
        load8f(dar + c * 8, dv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xh = (xv[j] - m) * r;
          const float gg = dv[j] * gm[i][j];
          s1 += gg;
          s2 += gg * xh;
          pg[i][j] += dv[j] * xh;
          pb[i][j] += dv[j];
        }
      }
    }
    const float2 sums = block_sum2(s1, s2, red);
    const float mean_g = sums.x * inv_h, mean_gx = sums.y * inv_h;
    const u16* dyr = dy + static_cast<size_t>(row) * h;
    u16* dxr = dx + static_cast<size_t>(row) * h;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * LNB_THREADS;
      if (c < nch) {
        float xv[8], dv[8], yv[8];
        unpack8(*reinterpret_cast<const uint4*>(xr + c * 8), xv);
        load8f(dar + c * 8, dv);
        unpack8(*reinterpret_cast<const uint4*>(dyr + c * 8), yv);
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int j0 = 2 * j, j1 = 2 * j + 1;
          const float v0 = yv[j0] + r * (dv[j0] * gm[i][j0] - mean_g - (xv[j0] - m) * r * mean_gx);
          const float v1 = yv[j1] + r * (dv[j1] * gm[i][j1] - mean_g - (xv[j1] - m) * r * mean_gx);
          o[j] = pack2bf(v0, v1);
        }
        *reinterpret_cast<uint4*>(dxr + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  float* pgr = partials + static_cast<size_t>(blockIdx.x) * 2 * h;
  float* pbr = pgr + h;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * LNB_THREADS;
    if (c < nch) {
#pragma unroll
      for (int j = 0; j < 8; j += 4) {
        *reinterpret_cast<float4*>(pgr + c * 8 + j) =
            make_float4(pg[i][j], pg[i][j + 1], pg[i][j + 2], pg[i][j + 3]);
        *reinterpret_cast<float4*>(pbr + c * 8 + j) =
            make_float4(pb[i][j], pb[i][j + 1], pb[i][j + 2], pb[i][j + 3]);
      }
    }
  }
}

// Sum the per-workgroup partials column by column.  A workgroup owns 64 of
// the 2h columns; its 4 waves each sum a quarter of the partial rows (lanes
// on consecutive columns: coalesced), then wave 0 adds the four quarters.
// The order is fixed, so the result is deterministic.
__global__ __launch_bounds__(256) void ln_bwd_reduce_kernel(const float* __restrict__ partials,
                                                            int nblk, int h,
                                                            u16* __restrict__ dgamma,
                                                            u16* __restrict__ dbeta) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  float acc = 0.0f;
  if (col < 2 * h)
    for (int b = wave; b < nblk; b += 4) acc += partials[static_cast<size_t>(b) * 2 * h + col];
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && col < 2 * h) {
    const float t = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
    if (col < h) dgamma[col] = f2bf(t);
    else dbeta[col - h] = f2bf(t);
  }
}

}  // namespace

hipError_t launch_layernorm_fwd(const u16* x, const u16* gamma, const u16* beta, u16* a,
                                u16* a_lo, float* mu, float* rstd, int T, int h, float eps,
                                hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(ln_fwd_kernel, dim3(T), dim3(LN_THREADS), 0, s, x, gamma, beta, a, a_lo,
                     mu, rstd, h, eps);
  return hipGetLastError();
}

int layernorm_bwd_blocks(int T) { return T < LN_BWD_BLOCKS ? (T < 1 ? 1 : T) : LN_BWD_BLOCKS; }

hipError_t launch_layernorm_bwd(const float* da, const u16* x, const u16* gamma,
                                const float* mu, const float* rstd, const u16* dy, u16* dx,
                                float* partials, u16* dgamma, u16* dbeta, int T, int h,
                                hipStream_t s) {
  const int nblk = layernorm_bwd_blocks(T);
  if (h <= 8 * LNB_THREADS)
    hipLaunchKernelGGL(ln_bwd_kernel<1>, dim3(nblk), dim3(LNB_THREADS), 0, s, da, x, gamma, mu,
                       rstd, dy, dx, partials, T, h);
  else
    hipLaunchKernelGGL(ln_bwd_kernel<2>, dim3(nblk), dim3(LNB_THREADS), 0, s, da, x, gamma, mu,
                       rstd, dy, dx, partials, T, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ln_bwd_reduce_kernel, dim3((2 * h + 63) / 64), dim3(256), 0, s, partials,
                     nblk, h, dgamma, dbeta);
  return hipGetLastError();
}

}  // namespace ptb
