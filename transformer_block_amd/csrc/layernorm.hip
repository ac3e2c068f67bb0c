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
// is written back in bf16 with 16-byte stores, together with an fp16 copy a16
// of the same fp32 values (used where bf16 rounding of a would be amplified:
// the query/key projection feeding the softmax logits, formed in fp16).
// Backward: each workgroup walks a strided set of rows (the next row's loads
// in flight while the current one is finished), computes
//   dx = dy + rstd * (g - mean(g) - xhat * mean(g * xhat)),  g = da * gamma,
// and keeps per-column partial sums of dgamma = sum da*xhat and dbeta = sum da
// in registers; a second kernel reduces the per-workgroup partials.
#include <algorithm>

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

// RMS: RMSNorm instead, a = gamma * x / sqrt(mean(x^2) + eps), no beta; the
// row mean is stored as 0 so that the backward's xhat = (x - mu) * rstd holds.
// clear[0, nclear) is set to zero on the way (the arrival counters of the
// launches that follow in the same stream), which saves a launch of its own.
template <bool RMS>
__global__ __launch_bounds__(LN_THREADS) void ln_fwd_kernel(const u16* __restrict__ x,
                                                            const u16* __restrict__ gamma,
                                                            const u16* __restrict__ beta,
                                                            u16* __restrict__ a,
                                                            u16* __restrict__ a16,
                                                            float* __restrict__ mu_out,
                                                            float* __restrict__ rstd_out,
                                                            int h, float eps,
                                                            int* __restrict__ clear, int nclear) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  for (int i = row * LN_THREADS + tid; i < nclear; i += static_cast<int>(gridDim.x) * LN_THREADS)
    clear[i] = 0;
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
  const float mu = RMS ? 0.0f : block_sum(sum, red) / static_cast<float>(h);
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
  u16* ahr = a16 != nullptr ? a16 + static_cast<size_t>(row) * h : nullptr;
#pragma unroll
  for (int i = 0; i < LN_MAXCH; ++i) {
    const int c = tid + i * LN_THREADS;
    if (c < nch) {
      float gm[8], bt[8];
      unpack8(*reinterpret_cast<const uint4*>(gamma + c * 8), gm);
      if (!RMS) unpack8(*reinterpret_cast<const uint4*>(beta + c * 8), bt);
      uint32_t o[4], oh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = (v[i][2 * j] - mu) * rstd * gm[2 * j] + (RMS ? 0.0f : bt[2 * j]);
        const float v1 = (v[i][2 * j + 1] - mu) * rstd * gm[2 * j + 1] + (RMS ? 0.0f : bt[2 * j + 1]);
        o[j] = pack2bf(v0, v1);
        oh[j] = pack2h(v0, v1);
      }
      *reinterpret_cast<uint4*>(ar + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      if (a16 != nullptr)
        *reinterpret_cast<uint4*>(ahr + c * 8) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
    }
  }
  if (tid == 0) { mu_out[row] = mu; rstd_out[row] = rstd; }
}

// dst[r][c] = fp16(src[r][c]) for a [rows, cols] block of a bf16 matrix
// (cols a multiple of 8, row strides ld_src and ld_dst in elements): the
// fp16 copy of the query/key columns of W_qkv for the fp16 q, k product.
// The block's 16-byte chunks are numbered row by row; workgroup g converts
// chunks [cpb g, cpb (g + 1)), thread t those at t + 256 u, all of its loads
// issued before the first store, consecutive threads on consecutive chunks.
// The launcher makes the grid one wave of the device's resident workgroups
// where the chunks allow, each with the same share to within one chunk per
// thread (no second, mostly idle wave of workgroups).
// The conversion is exact for every bf16 value inside the fp16 normal range;
// smaller magnitudes round to fp16 subnormals (absolute error <= 2^-25) and
// larger ones saturate at 65504.
constexpr int CAST_MAX_PER = 10;  // chunks per thread at most
__global__ __launch_bounds__(256) void cast_f16_kernel(const u16* __restrict__ src, int ld_src,
                                                       u16* __restrict__ dst, int ld_dst,
                                                       int rows, int cols8, int cpb) {
  const int total = rows * cols8;  // < 2^31 (checked by the launcher)
  const int first = blockIdx.x * cpb, len = min(cpb, total - first);
  uint4 v[CAST_MAX_PER];
  int off[CAST_MAX_PER];  // destination element offset, -1 past the block
#pragma unroll
  for (int u = 0; u < CAST_MAX_PER; ++u) {
    const int rel = static_cast<int>(threadIdx.x) + 256 * u;
    off[u] = -1;
    if (rel < len) {
      const int idx = first + rel;
      const int r = idx / cols8, c = idx - r * cols8;
      v[u] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r) * ld_src + c * 8);
      off[u] = r * ld_dst + c * 8;
    }
  }
#pragma unroll
  for (int u = 0; u < CAST_MAX_PER; ++u) {
    if (off[u] >= 0) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&v[u]);
      uint4 o;
      o.x = pack2h(lo_bf(w[0]), hi_bf(w[0]));
      o.y = pack2h(lo_bf(w[1]), hi_bf(w[1]));
      o.z = pack2h(lo_bf(w[2]), hi_bf(w[2]));
      o.w = pack2h(lo_bf(w[3]), hi_bf(w[3]));
      *reinterpret_cast<uint4*>(dst + off[u]) = o;
    }
  }
}

constexpr int LNB_THREADS = 512;  // 8 waves: two per SIMD, up to 256 VGPRs each
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

// One row of the backward's inputs as this thread holds them: NCH 16-byte
// chunks (8 bf16 each) of x, dy and da, plus the row's statistics.
template <int NCH>
struct LnRow {
  uint4 x[NCH], dy[NCH], da[NCH];
  float mu, rstd;
};

template <int NCH>
__device__ __forceinline__ void load_row(LnRow<NCH>& d, const u16* da, const u16* x,
                                         const u16* dy, const float* mu, const float* rstd,
                                         int row, int h, int nch) {
  d.mu = mu[row];
  d.rstd = rstd[row];
  const size_t base = static_cast<size_t>(row) * h;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + i * LNB_THREADS;
    if (c < nch) {
      d.x[i] = *reinterpret_cast<const uint4*>(x + base + c * 8);
      d.da[i] = *reinterpret_cast<const uint4*>(da + base + c * 8);
      d.dy[i] = *reinterpret_cast<const uint4*>(dy + base + c * 8);
    }
  }
}

// NCH = 16-byte chunks of a row per thread (h <= NCH * 8 * 512).  RMS: the
// RMSNorm backward, dx = dy + rstd * (g - xhat * mean(g * xhat)) (no mean(g)
// term; xhat = x * rstd from the stored mean 0), and dbeta = 0.  Each row is
// read once, into registers, and the next row of the workgroup is loaded
// while the current one is reduced and written, so a workgroup always has a
// row's worth of loads in flight (two rows of registers).
template <int NCH, bool RMS>
__global__ __launch_bounds__(LNB_THREADS) void ln_bwd_kernel(
    const u16* __restrict__ da, const u16* __restrict__ x, const u16* __restrict__ gamma,
    const float* __restrict__ mu, const float* __restrict__ rstd, const u16* __restrict__ dy,
    u16* __restrict__ dx, float* __restrict__ partials, int T, int h) {
  __shared__ float red[2 * LNB_WAVES];
  const int tid = threadIdx.x;
  const int nch = h >> 3;
  const float inv_h = 1.0f / static_cast<float>(h);
  uint4 gmp[NCH];  // gamma, packed: unpacked where used
  float pg[NCH][8], pb[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * LNB_THREADS;
#pragma unroll
    for (int j = 0; j < 8; ++j) { pg[i][j] = 0.0f; pb[i][j] = 0.0f; }
    gmp[i] = c < nch ? *reinterpret_cast<const uint4*>(gamma + c * 8) : make_uint4(0, 0, 0, 0);
  }
  LnRow<NCH> cur;
  int row = blockIdx.x;
  if (row < T) load_row(cur, da, x, dy, mu, rstd, row, h, nch);
  for (; row < T; row += gridDim.x) {
    LnRow<NCH> nxt;
    if (row + static_cast<int>(gridDim.x) < T)
      load_row(nxt, da, x, dy, mu, rstd, row + gridDim.x, h, nch);
    const float m = cur.mu, r = cur.rstd;
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * LNB_THREADS;
      if (c < nch) {
        float xv[8], gm[8], dv[8];
        unpack8(cur.x[i], xv);
        unpack8(gmp[i], gm);
        unpack8(cur.da[i], dv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xh = (xv[j] - m) * r;
          const float gg = dv[j] * gm[j];
          s1 += gg;
          s2 += gg * xh;
          pg[i][j] += dv[j] * xh;
          if (!RMS) pb[i][j] += dv[j];
        }
      }
    }
    const float2 sums = block_sum2(s1, s2, red);
    const float mean_g = RMS ? 0.0f : sums.x * inv_h, mean_gx = sums.y * inv_h;
    u16* dxr = dx + static_cast<size_t>(row) * h;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * LNB_THREADS;
      if (c < nch) {
        float xv[8], gm[8], yv[8], dv[8];
        unpack8(cur.da[i], dv);
        unpack8(cur.x[i], xv);
        unpack8(gmp[i], gm);
        unpack8(cur.dy[i], yv);
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int j0 = 2 * j, j1 = 2 * j + 1;
          const float v0 = yv[j0] + r * (dv[j0] * gm[j0] - mean_g - (xv[j0] - m) * r * mean_gx);
          const float v1 = yv[j1] + r * (dv[j1] * gm[j1] - mean_g - (xv[j1] - m) * r * mean_gx);
          o[j] = pack2bf(v0, v1);
        }
        *reinterpret_cast<uint4*>(dxr + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    cur = nxt;
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

// Sum the per-workgroup partials column by column.  A workgroup owns 256 of
// the 2h columns (64 lanes x 4 consecutive columns, 16-byte loads); its 8
// waves each sum every 8th partial row, then wave 0 adds the eight in a fixed
// order, so the result is deterministic.
constexpr int LNR_WAVES = 8;
__global__ __launch_bounds__(64 * LNR_WAVES) void ln_bwd_reduce_kernel(
    const float* __restrict__ partials, int nblk, int h, u16* __restrict__ dgamma,
    u16* __restrict__ dbeta) {
  __shared__ float4 part[LNR_WAVES][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c4 = blockIdx.x * 64 + lane;  // float4 column
  const int n4 = h / 2;                   // 2h columns in float4s
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (c4 < n4) {
#pragma unroll 8
    for (int b = wave; b < nblk; b += LNR_WAVES) {
      const float4 v = reinterpret_cast<const float4*>(partials + static_cast<size_t>(b) * 2 * h)[c4];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && c4 < n4) {
    float4 t = part[0][lane];
#pragma unroll
    for (int w = 1; w < LNR_WAVES; ++w) {
      const float4 v = part[w][lane];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    const int col = 4 * c4;  // h is a multiple of 4: the four columns lie on one side
    u16* o = col < h ? dgamma + col : dbeta + (col - h);
    const uint2 packed = make_uint2(pack2bf(t.x, t.y), pack2bf(t.z, t.w));
    *reinterpret_cast<uint2*>(o) = packed;
  }
}

}  // namespace

hipError_t launch_layernorm_fwd(const u16* x, const u16* gamma, const u16* beta, u16* a,
                                u16* a16, float* mu, float* rstd, int T, int h, float eps,
                                hipStream_t s, bool rms, int* clear, int nclear) {
  if (clear == nullptr || nclear < 0) nclear = 0;
  if (T <= 0) return launch_zero_i32(clear, nclear, s);
  hipLaunchKernelGGL(rms ? ln_fwd_kernel<true> : ln_fwd_kernel<false>, dim3(T), dim3(LN_THREADS),
                     0, s, x, gamma, beta, a, a16, mu, rstd, h, eps, clear, nclear);
  return hipGetLastError();
}

hipError_t launch_cast_f16(const u16* src, int ld_src, int rows, int cols, u16* dst, int ld_dst,
                           hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 8 != 0 || ld_src % 8 != 0 || ld_dst % 8 != 0 || ld_src < cols || ld_dst < cols ||
      static_cast<long>(rows) * ld_dst >= (1L << 31) || static_cast<long>(rows) * (cols / 8) >= (1L << 31))
    return hipErrorInvalidValue;
  const long chunks = static_cast<long>(rows) * (cols / 8);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cast_f16_kernel, 256, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int cus = device_compute_units();
  const long slots = static_cast<long>(per_cu) * (cus > 0 ? cus : 256);
  // one wave of workgroups if each thread's share stays within CAST_MAX_PER
  // chunks, else as many full workgroups as that takes
  const long blocks = std::max<long>(std::min<long>(slots, (chunks + 255) / 256),
                                     (chunks + 256L * CAST_MAX_PER - 1) / (256L * CAST_MAX_PER));
  const long cpb = (chunks + blocks - 1) / blocks;  // <= 256 * CAST_MAX_PER
  hipLaunchKernelGGL(cast_f16_kernel, dim3(static_cast<unsigned>((chunks + cpb - 1) / cpb)), dim3(256),
                     0, s, src, ld_src, dst, ld_dst, rows, cols / 8, static_cast<int>(cpb));
  return hipGetLastError();
}

int layernorm_bwd_blocks(int T) { return T < LN_BWD_BLOCKS ? (T < 1 ? 1 : T) : LN_BWD_BLOCKS; }

hipError_t launch_layernorm_bwd(const u16* da, const u16* x, const u16* gamma,
                                const float* mu, const float* rstd, const u16* dy, u16* dx,
                                float* partials, u16* dgamma, u16* dbeta, int T, int h,
                                hipStream_t s, bool rms) {
  const int nblk = layernorm_bwd_blocks(T);
  auto* kern = h <= 8 * LNB_THREADS    ? (rms ? ln_bwd_kernel<1, true> : ln_bwd_kernel<1, false>)
               : h <= 16 * LNB_THREADS ? (rms ? ln_bwd_kernel<2, true> : ln_bwd_kernel<2, false>)
               : h <= 24 * LNB_THREADS ? (rms ? ln_bwd_kernel<3, true> : ln_bwd_kernel<3, false>)
                                       : (rms ? ln_bwd_kernel<4, true> : ln_bwd_kernel<4, false>);
  hipLaunchKernelGGL(kern, dim3(nblk), dim3(LNB_THREADS), 0, s, da, x, gamma, mu, rstd, dy, dx,
                     partials, T, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ln_bwd_reduce_kernel, dim3((h / 2 + 63) / 64), dim3(64 * LNR_WAVES), 0, s,
                     partials, nblk, h, dgamma, dbeta);
  return hipGetLastError();
}

}  // namespace ptb
