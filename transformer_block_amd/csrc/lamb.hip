// LAMB optimizer step for gfx950 (MegaScale reading notes, section 1.1,
// eq (7)): per parameter tensor ("layer" l),
//   m_l <- b1 m_l + (1 - b1) g_l,   v_l <- b2 v_l + (1 - b2) g_l^2,
//   r_l  = (m_l / (1 - b1^t)) / (sqrt(v_l / (1 - b2^t)) + eps),
//   theta_l <- theta_l - lr * (||theta_l|| / ||r_l||) * r_l,
// with fp32 master weights and moments (Megatron tuning post, mixed-precision
// section: low-precision compute, fp32 master copy and optimizer update) and
// the bf16 copy of theta the next forward reads written alongside.
//
// HBM-bound, three launches over every tensor of one call:
//   1. moments: read g (bf16), theta, m, v; write m, v; per-workgroup partial
//      sums of theta^2 and r^2 (fp32 per thread, fp64 across the workgroup);
//   2. norms: one workgroup per tensor sums its partials in a fixed order;
//   3. update: recompute r from the new m, v (the same fp32 operations give
//      the same r), theta -= lr * trust * r; write theta and bf16(theta).
// Every thread moves 8 consecutive elements per iteration with 16-byte
// accesses.  Results do not depend on timing (fixed reduction order).
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

// Static scratch of the allocation-free step (launch_lamb with the pointer
// from lamb_static_scratch): each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes this name to a kernel (in
// host code it is a stand-in, not a device address): the per-device address
// comes from hipGetSymbolAddress.
static __device__ __align__(256) double scratch[kLambStaticScratchBytes / sizeof(double)];

constexpr int LAMB_THREADS = 256;
constexpr int LAMB_VEC = 8;                                      // elements per thread per pass
constexpr int LAMB_ITERS = 8;                                    // passes per workgroup
constexpr int LAMB_CHUNK = LAMB_THREADS * LAMB_VEC * LAMB_ITERS;  // 16384 elements

struct LambArgs {
  float* theta[kLambMaxTensors];
  float* m[kLambMaxTensors];
  float* v[kLambMaxTensors];
  const u16* g[kLambMaxTensors];
  u16* w[kLambMaxTensors];
  long numel[kLambMaxTensors];
  int block0[kLambMaxTensors + 1];  // first workgroup of each tensor; [n] = total
  int n;
  float lr, b1, b2, eps, inv_bc1, inv_bc2;
  double* partial;  // [total workgroups][2]: sum theta^2, sum r^2
  float* norms;     // [n][2]: ||theta||, ||r||
};

__device__ __forceinline__ int tensor_of(const LambArgs& a, int blk) {
  int t = 0;
  while (t + 1 < a.n && a.block0[t + 1] <= blk) ++t;
  return t;
}

__device__ __forceinline__ void load8f(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8f(float* p, const float* x) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// r for one element from the updated moments (the same operations in both
// passes, so pass 3 reproduces pass 1's r exactly)
__device__ __forceinline__ float lamb_dir(float m, float v, const LambArgs& a) {
  return (m * a.inv_bc1) / (sqrtf(v * a.inv_bc2) + a.eps);
}

__global__ __launch_bounds__(LAMB_THREADS) void lamb_moments_kernel(LambArgs a) {
  const int blk = blockIdx.x;
  const int t = tensor_of(a, blk);
  const long base = static_cast<long>(blk - a.block0[t]) * LAMB_CHUNK;
  const long n = a.numel[t];
  float st = 0.0f, sr = 0.0f;
  for (int it = 0; it < LAMB_ITERS; ++it) {
    const long e = base + (static_cast<long>(it) * LAMB_THREADS + threadIdx.x) * LAMB_VEC;
    if (e >= n) break;
    float th[8], mm[8], vv[8], gg[8];
    load8f(a.theta[t] + e, th);
    load8f(a.m[t] + e, mm);
    load8f(a.v[t] + e, vv);
    const uint4 gw = *reinterpret_cast<const uint4*>(a.g[t] + e);
    const uint32_t gu[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { gg[2 * i] = lo_bf(gu[i]); gg[2 * i + 1] = hi_bf(gu[i]); }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mm[i] = a.b1 * mm[i] + (1.0f - a.b1) * gg[i];
      vv[i] = a.b2 * vv[i] + (1.0f - a.b2) * (gg[i] * gg[i]);
      const float r = lamb_dir(mm[i], vv[i], a);
      st += th[i] * th[i];
      sr += r * r;
    }
    store8f(a.m[t] + e, mm);
    store8f(a.v[t] + e, vv);
  }
  // workgroup sums in fp64 (fixed order)
  __shared__ double red[2][LAMB_THREADS / 64];
  double dt = st, dr = sr;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) { dt += __shfl_xor(dt, o); dr += __shfl_xor(dr, o); }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = dt; red[1][wave] = dr; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s0 = 0.0, s1 = 0.0;
    for (int w = 0; w < LAMB_THREADS / 64; ++w) { s0 += red[0][w]; s1 += red[1][w]; }
    a.partial[2 * blk] = s0;
    a.partial[2 * blk + 1] = s1;
  }
}

__global__ __launch_bounds__(LAMB_THREADS) void lamb_norms_kernel(LambArgs a) {
  const int t = blockIdx.x;
  const int b0 = a.block0[t], b1 = a.block0[t + 1];
  double s0 = 0.0, s1 = 0.0;
  for (int b = b0 + static_cast<int>(threadIdx.x); b < b1; b += LAMB_THREADS) {
    s0 += a.partial[2 * b];
    s1 += a.partial[2 * b + 1];
  }
  __shared__ double red[2][LAMB_THREADS];
  red[0][threadIdx.x] = s0;
  red[1][threadIdx.x] = s1;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t0 = 0.0, t1 = 0.0;
    for (int i = 0; i < LAMB_THREADS; ++i) { t0 += red[0][i]; t1 += red[1][i]; }
    a.norms[2 * t] = static_cast<float>(sqrt(t0));
    a.norms[2 * t + 1] = static_cast<float>(sqrt(t1));
  }
}

__global__ __launch_bounds__(LAMB_THREADS) void lamb_update_kernel(LambArgs a) {
  const int blk = blockIdx.x;
  const int t = tensor_of(a, blk);
  const long base = static_cast<long>(blk - a.block0[t]) * LAMB_CHUNK;
  const long n = a.numel[t];
  const float nt = a.norms[2 * t], nr = a.norms[2 * t + 1];
  // a tensor whose weights or direction are all zero takes the plain step
  const float trust = (nt > 0.0f && nr > 0.0f) ? nt / nr : 1.0f;
  const float scale = a.lr * trust;
  for (int it = 0; it < LAMB_ITERS; ++it) {
    const long e = base + (static_cast<long>(it) * LAMB_THREADS + threadIdx.x) * LAMB_VEC;
    if (e >= n) break;
    float th[8], mm[8], vv[8];
    load8f(a.theta[t] + e, th);
    load8f(a.m[t] + e, mm);
    load8f(a.v[t] + e, vv);
#pragma unroll
    for (int i = 0; i < 8; ++i) th[i] -= scale * lamb_dir(mm[i], vv[i], a);
    store8f(a.theta[t] + e, th);
    uint4 wb;
    wb.x = pack2bf(th[0], th[1]); wb.y = pack2bf(th[2], th[3]);
    wb.z = pack2bf(th[4], th[5]); wb.w = pack2bf(th[6], th[7]);
    *reinterpret_cast<uint4*>(a.w[t] + e) = wb;
  }
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
double* scratch_ptr[kMaxDevices];  // guarded by scratch_mutex

}  // namespace

hipError_t lamb_static_scratch(double** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = static_cast<double*>(p);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

int lamb_blocks(long numel) { return static_cast<int>((numel + LAMB_CHUNK - 1) / LAMB_CHUNK); }

hipError_t launch_lamb(const LambTensor* ts, int n, const LambHyper& hp, double* partial,
                       float* norms, hipStream_t s) {
  if (n < 1 || n > kLambMaxTensors) return hipErrorInvalidValue;
  LambArgs a;
  int blocks = 0;
  for (int i = 0; i < n; ++i) {
    a.theta[i] = ts[i].theta; a.m[i] = ts[i].m; a.v[i] = ts[i].v;
    a.g[i] = ts[i].grad; a.w[i] = ts[i].weight; a.numel[i] = ts[i].numel;
    a.block0[i] = blocks;
    blocks += lamb_blocks(ts[i].numel);
  }
  for (int i = n; i <= kLambMaxTensors; ++i) a.block0[i] = blocks;
  a.n = n;
  a.lr = hp.lr; a.b1 = hp.beta1; a.b2 = hp.beta2; a.eps = hp.eps;
  a.inv_bc1 = static_cast<float>(1.0 / (1.0 - pow(static_cast<double>(hp.beta1), hp.step)));
  a.inv_bc2 = static_cast<float>(1.0 / (1.0 - pow(static_cast<double>(hp.beta2), hp.step)));
  a.partial = partial;
  a.norms = norms;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(lamb_moments_kernel, dim3(blocks), dim3(LAMB_THREADS), 0, s, a);
  hipLaunchKernelGGL(lamb_norms_kernel, dim3(n), dim3(LAMB_THREADS), 0, s, a);
  hipLaunchKernelGGL(lamb_update_kernel, dim3(blocks), dim3(LAMB_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace ptb
