// Current-scaling FP8 casts (Megatron-LM tuning post, mixed-precision
// section: E4M3 / E5M2 operands for the matrix products, the scale of a
// tensor taken from the tensor itself).
//
//   amax:  max |x| over a logical bf16 matrix (one or two unpadded
//          segments), one workgroup per CU walking them as flat arrays, one
//          vector atomic max per workgroup on the float's bits (non-negative
//          floats order like their bit patterns).
//   cast:  code = RNE(clamp(x * s, -FMAX, FMAX)) with s = FMAX / amax, x * s
//          one fp32 multiply; written row-wise (same layout) and/or
//          transposed, so that every FP8 product reads two k-contiguous
//          operands.  Tiles of 64 rows x 128 columns: each thread converts a
//          4 x 8 block from four 16-byte loads; the transpose goes through
//          LDS as 4-byte columns of codes and leaves as 16-byte rows.
//          Padding (up to the output's leading dimension) is written as zero
//          codes, so that products can run K up to a whole number of
//          128-wide k-steps.
//   mx:    block scaling (mxfp8): the same tiles, each copy quantized on
//          blocks of 32 along its own contiguous dimension, so the row-wise
//          and the transposed copy get codes and scales of their own.  A
//          row's block maximum comes from a 4-lane shuffle (32 columns = 4
//          threads); a column's from a shuffle over the wave's 16 rows and
//          one LDS exchange between the two waves of a 32-row block.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int CR = 64;        // cast tile: rows of X
constexpr int CC = 128;       // cast tile: columns of X
constexpr int TSW = CR / 4 + 1;  // LDS words per transposed row (64 codes + 4 bytes of pad)

__device__ __forceinline__ const u16* src_at(const CastSrc& x, int r, int c) {
  if (x.split_on_rows)
    return r < x.split ? x.p0 + static_cast<size_t>(r) * x.ld0 + c
                       : x.p1 + static_cast<size_t>(r - x.split) * x.ld1 + c;
  return c < x.split ? x.p0 + static_cast<size_t>(r) * x.ld0 + c
                     : x.p1 + static_cast<size_t>(r) * x.ld1 + (c - x.split);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

constexpr int AMAX_THREADS = 1024;
constexpr int AMAX_UNROLL = 8;  // 16-byte loads in flight per thread

// max |x| over up to two contiguous arrays of n0 and n1 16-byte chunks (the
// segments of a logical matrix without padding): a grid-stride walk in which
// consecutive threads read consecutive chunks, eight in flight each.  The
// grid is one workgroup per CU: the workgroups' one atomic each all go to
// the same address and are served one at a time (a grid of 1024 workgroups
// spent a third of an activation's amax on them).
__global__ __launch_bounds__(AMAX_THREADS) void amax_flat_kernel(const uint4* p0, long n0,
                                                                 const uint4* p1, long n1,
                                                                 float* amax) {
  __shared__ uint32_t part[AMAX_THREADS / 64];
  uint32_t m = 0;
  const long stride = static_cast<long>(gridDim.x) * AMAX_THREADS;
#pragma unroll
  for (int seg = 0; seg < 2; ++seg) {
    const uint4* p = seg ? p1 : p0;
    const long n = seg ? n1 : n0;
    for (long i0 = static_cast<long>(blockIdx.x) * AMAX_THREADS + threadIdx.x; i0 < n;
         i0 += AMAX_UNROLL * stride) {
      uint4 v[AMAX_UNROLL];
#pragma unroll
      for (int u = 0; u < AMAX_UNROLL; ++u) {
        const long i = i0 + u * stride;
        v[u] = i < n ? p[i] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < AMAX_UNROLL; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          m = umax(m, (w[k] & 0x7fffu) << 16);
          m = umax(m, w[k] & 0x7fff0000u);
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = umax(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < AMAX_THREADS / 64; ++w) m = umax(m, part[w]);
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

// One tile of X, CR rows x CC columns at (r0, c0).  Thread (br, bc) =
// (tid / 16, tid % 16) owns rows r0 + 4 br .. +3 and columns c0 + 8 bc .. +7
// (four 16-byte loads).  Codes go out row-wise as 8-byte stores; for the
// transpose each thread writes its 8 columns x 4 rows into LDS as 4-byte
// column pieces, and each output row of 64 codes leaves as two 16-byte
// stores from a pair of threads.
template <int FMT>
__global__ __launch_bounds__(256) void cast_kernel(CastSrc x, const float* amax, uint8_t* rows,
                                                   int ldr, uint8_t* cols, int ldc) {
  __shared__ uint32_t tt[CC * TSW];
  const float s = fp8_scale(*amax, fp8_max(FMT));
  const int r0 = blockIdx.y * CR, c0 = blockIdx.x * CC;
  const int tid = threadIdx.x, br = tid >> 4, bc = tid & 15;
  const int c = c0 + 8 * bc;
  uint2 q[4];  // q[i]: codes of row r0 + 4 br + i, columns c .. c+7
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 4 * br + i;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < x.R && c < x.C) v = *reinterpret_cast<const uint4*>(src_at(x, r, c));
    q[i].x = quant4<FMT>(lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y), s);
    q[i].y = quant4<FMT>(lo_bf(v.z), hi_bf(v.z), lo_bf(v.w), hi_bf(v.w), s);
  }
  if (rows != nullptr && c < ldr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 4 * br + i;
      if (r < x.R) *reinterpret_cast<uint2*>(rows + static_cast<size_t>(r) * ldr + c) = q[i];
    }
  }
  if (cols == nullptr || r0 >= ldc) return;
  // column j of the thread's block: rows 4 br .. +3 as one 4-byte word
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int sh = 8 * (j & 3);
    const uint32_t w0 = j < 4 ? q[0].x : q[0].y, w1 = j < 4 ? q[1].x : q[1].y;
    const uint32_t w2 = j < 4 ? q[2].x : q[2].y, w3 = j < 4 ? q[3].x : q[3].y;
    tt[(8 * bc + j) * TSW + br] = ((w0 >> sh) & 0xffu) | (((w1 >> sh) & 0xffu) << 8) |
                                  (((w2 >> sh) & 0xffu) << 16) | (((w3 >> sh) & 0xffu) << 24);
  }
  __syncthreads();
  // output row oc = column c0 + oc of X, codes of rows r0 + 32 (tid % 2) .. +31
  const int oc = tid >> 1, ow = (tid & 1) * 8;
  if (c0 + oc >= x.C) return;
  const uint32_t* t = tt + oc * TSW + ow;
  uint8_t* o = cols + static_cast<size_t>(c0 + oc) * ldc + r0 + ow * 4;
  reinterpret_cast<uint4*>(o)[0] = make_uint4(t[0], t[1], t[2], t[3]);
  reinterpret_cast<uint4*>(o)[1] = make_uint4(t[4], t[5], t[6], t[7]);
}

// E8M0 scale code of a block whose largest magnitude has the bf16 bits m
// (sign cleared): 127 + floor(log2 amax) - emax, within 0..254; 127 (scale 1)
// for an all-zero block.
template <int FMT>
__device__ __forceinline__ uint32_t mx_code(uint32_t m) {
  constexpr int EMAX = FMT == FP8_E4M3 ? 8 : 15;
  if (m == 0) return 127u;
  const int e = static_cast<int>(m >> 7);
  const int fl = e != 0 ? e - 127 : (31 - __clz(static_cast<int>(m))) - 133;  // subnormal: m 2^-133
  return static_cast<uint32_t>(min(max(fl - EMAX + 127, 0), 254));
}

// 2^-X for scale code c (X = c - 127); exact, never subnormal for the codes
// a finite bf16 block produces.
__device__ __forceinline__ float mx_mult(uint32_t c) {
  return __builtin_amdgcn_ldexpf(1.0f, 127 - static_cast<int>(c));
}

// One tile of X as cast_kernel, block-scaled.  Thread (br, bc) owns rows
// r0 + 4 br .. +3 and columns c0 + 8 bc .. +7.  Row-wise: the 32-column
// block of a row spans threads bc & ~3 .. +3; threads bc = 0 collect the four
// block codes of their rows (the tile is one k-step) and write them where
// mx_scale_byte puts them.
// Transposed: the 32-row block of a column spans waves 2 blk and 2 blk + 1;
// each wave reduces its 16 rows by shuffles and leaves the column maxima in
// LDS.
template <int FMT>
__global__ __launch_bounds__(256) void mx_cast_kernel(CastSrc x, uint8_t* rows, int ldr,
                                                      uint32_t* rs, int rs_ld, uint8_t* cols,
                                                      int ldc, uint32_t* cs, int cs_ld) {
  __shared__ uint32_t tt[CC * TSW];
  __shared__ uint32_t cmax[4 * CC];  // [wave][column]: max |x| bits over the wave's 16 rows
  const int r0 = blockIdx.y * CR, c0 = blockIdx.x * CC;
  const int tid = threadIdx.x, br = tid >> 4, bc = tid & 15, wave = tid >> 6, lane = tid & 63;
  const int c = c0 + 8 * bc;
  uint32_t w[4][4];  // w[i][j/2]: bf16 pair of row r0 + 4 br + i, columns c + j, c + j + 1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 4 * br + i;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < x.R && c < x.C) v = *reinterpret_cast<const uint4*>(src_at(x, r, c));
    w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
  }
  auto mag = [&](int i, int j) { return (w[i][j >> 1] >> (16 * (j & 1))) & 0x7fffu; };
  auto val = [&](int i, int j) { return (j & 1) ? hi_bf(w[i][j >> 1]) : lo_bf(w[i][j >> 1]); };
  auto xmax = [](uint32_t m, int o) {
    return umax(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
  };

  if (rows != nullptr && c0 < ldr) {
    uint32_t code[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = umax(m, mag(i, j));
      m = xmax(xmax(m, 1), 2);
      code[i] = mx_code<FMT>(m);
      const float s = mx_mult(code[i]);
      uint2 q;
      q.x = quant4<FMT>(val(i, 0), val(i, 1), val(i, 2), val(i, 3), s);
      q.y = quant4<FMT>(val(i, 4), val(i, 5), val(i, 6), val(i, 7), s);
      const int r = r0 + 4 * br + i;
      if (r < x.R) *reinterpret_cast<uint2*>(rows + static_cast<size_t>(r) * ldr + c) = q;
    }
    uint32_t blk[4][4];  // [row i][block b]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        blk[i][b] = static_cast<uint32_t>(__shfl(static_cast<int>(code[i]), lane + 4 * b));
    if (bc == 0 && r0 < rs_ld) {
      uint8_t* sb = reinterpret_cast<uint8_t*>(rs);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          sb[mx_scale_byte(c0 / CC, r0 + 4 * br + i, b, rs_ld)] = static_cast<uint8_t>(blk[i][b]);
    }
  }
  if (cols == nullptr || r0 >= ldc) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t m = umax(umax(mag(0, j), mag(1, j)), umax(mag(2, j), mag(3, j)));
    m = xmax(xmax(m, 16), 32);
    if (lane < 16) cmax[wave * CC + 8 * bc + j] = m;
  }
  __syncthreads();
  const int blk = wave >> 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = 8 * bc + j;
    const float s = mx_mult(mx_code<FMT>(umax(cmax[2 * blk * CC + col], cmax[(2 * blk + 1) * CC + col])));
    tt[col * TSW + br] = quant4<FMT>(val(0, j), val(1, j), val(2, j), val(3, j), s);
  }
  if (tid < CC && c0 + tid < cs_ld) {
    // this tile's two k-blocks of column c0 + tid: blocks (r0 % 128) / 32 + 0, 1
    uint8_t* sb = reinterpret_cast<uint8_t*>(cs);
    const int b0 = (r0 % 128) / 32;
    sb[mx_scale_byte(r0 / 128, c0 + tid, b0, cs_ld)] =
        static_cast<uint8_t>(mx_code<FMT>(umax(cmax[tid], cmax[CC + tid])));
    sb[mx_scale_byte(r0 / 128, c0 + tid, b0 + 1, cs_ld)] =
        static_cast<uint8_t>(mx_code<FMT>(umax(cmax[2 * CC + tid], cmax[3 * CC + tid])));
  }
  __syncthreads();
  const int oc = tid >> 1, ow = (tid & 1) * 8;
  if (c0 + oc >= x.C) return;
  const uint32_t* t = tt + oc * TSW + ow;
  uint8_t* o = cols + static_cast<size_t>(c0 + oc) * ldc + r0 + ow * 4;
  reinterpret_cast<uint4*>(o)[0] = make_uint4(t[0], t[1], t[2], t[3]);
  reinterpret_cast<uint4*>(o)[1] = make_uint4(t[4], t[5], t[6], t[7]);
}

bool src_ok(const CastSrc& x) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  return x.p0 != nullptr && x.p1 != nullptr && al(x.p0) && al(x.p1) && x.R > 0 && x.C > 0 &&
         x.C % 8 == 0 && x.ld0 % 8 == 0 && x.ld1 % 8 == 0 && x.split % 8 == 0 && x.split > 0;
}

}  // namespace

hipError_t launch_amax(const CastSrc& x, float* amax, hipStream_t s) {
  if (!src_ok(x) || amax == nullptr) return hipErrorInvalidValue;
  int cus = device_compute_units();
  if (cus <= 0) cus = 256;
  // the segments must be plain arrays (leading dimension = segment width)
  const bool one = x.split_on_rows ? x.split >= x.R : x.split >= x.C;
  const long R0 = x.split_on_rows && !one ? x.split : x.R;
  const long C0 = !x.split_on_rows && !one ? x.split : x.C;
  const long R1 = one ? 0 : (x.split_on_rows ? x.R - x.split : x.R);
  const long C1 = one ? 0 : (x.split_on_rows ? x.C : x.C - x.split);
  if (x.ld0 != C0 || (!one && x.ld1 != C1)) return hipErrorInvalidValue;
  const long n0 = R0 * C0 / 8, n1 = R1 * C1 / 8;
  const int blocks =
      static_cast<int>(std::min<long>((n0 + n1 + AMAX_THREADS - 1) / AMAX_THREADS, cus));
  hipLaunchKernelGGL(amax_flat_kernel, dim3(blocks), dim3(AMAX_THREADS), 0, s,
                     reinterpret_cast<const uint4*>(x.p0), n0,
                     reinterpret_cast<const uint4*>(x.p1), n1, amax);
  return hipGetLastError();
}

hipError_t launch_cast_fp8(const CastSrc& x, Fp8Format fmt, const float* amax, uint8_t* rows,
                           int ldr, uint8_t* cols, int ldc, hipStream_t s) {
  if (!src_ok(x) || amax == nullptr || (rows == nullptr && cols == nullptr))
    return hipErrorInvalidValue;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (rows != nullptr && (ldr < x.C || ldr % 64 != 0 || !al(rows))) return hipErrorInvalidValue;
  if (cols != nullptr && (ldc < x.R || ldc % 64 != 0 || !al(cols))) return hipErrorInvalidValue;
  const int rspan = cols != nullptr ? std::max(x.R, ldc) : x.R;
  const int cspan = rows != nullptr ? std::max(x.C, ldr) : x.C;
  const dim3 grid((cspan + CC - 1) / CC, (rspan + CR - 1) / CR);
  if (fmt == FP8_E4M3)
    hipLaunchKernelGGL(cast_kernel<FP8_E4M3>, grid, dim3(256), 0, s, x, amax, rows, ldr, cols, ldc);
  else
    hipLaunchKernelGGL(cast_kernel<FP8_E5M2>, grid, dim3(256), 0, s, x, amax, rows, ldr, cols, ldc);
  return hipGetLastError();
}

hipError_t launch_cast_mx(const CastSrc& x, Fp8Format fmt, uint8_t* rows, int ldr, uint32_t* rs,
                          int rs_ld, uint8_t* cols, int ldc, uint32_t* cs, int cs_ld,
                          hipStream_t s) {
  if (!src_ok(x) || (rows == nullptr && cols == nullptr)) return hipErrorInvalidValue;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (rows != nullptr && (ldr < x.C || ldr % CC != 0 || !al(rows) || rs == nullptr || !al(rs) ||
                          rs_ld < x.R || rs_ld % 128 != 0))
    return hipErrorInvalidValue;
  if (cols != nullptr && (ldc < x.R || ldc % CC != 0 || !al(cols) || cs == nullptr || !al(cs) ||
                          cs_ld < x.C || cs_ld % 128 != 0))
    return hipErrorInvalidValue;
  // tiles over every code and scale word either copy holds (padding included)
  int rspan = x.R, cspan = x.C;
  if (rows != nullptr) { cspan = std::max(cspan, ldr); rspan = std::max(rspan, rs_ld); }
  if (cols != nullptr) { rspan = std::max(rspan, ldc); cspan = std::max(cspan, cs_ld); }
  const dim3 grid((cspan + CC - 1) / CC, (rspan + CR - 1) / CR);
  if (fmt == FP8_E4M3)
    hipLaunchKernelGGL(mx_cast_kernel<FP8_E4M3>, grid, dim3(256), 0, s, x, rows, ldr, rs, rs_ld,
                       cols, ldc, cs, cs_ld);
  else
    hipLaunchKernelGGL(mx_cast_kernel<FP8_E5M2>, grid, dim3(256), 0, s, x, rows, ldr, rs, rs_ld,
                       cols, ldc, cs, cs_ld);
  return hipGetLastError();
}

}  // namespace ptb
