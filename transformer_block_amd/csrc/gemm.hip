// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16) with LDS-staged,
// double-buffered tiles and fused epilogues.
//
// One kernel template covers the six matrix products of the Parallel
// Transformer Block layer (MegaScale reading notes, section 1.1, eq (4); fused
// QKV projection, section 1.3; MLP Y = GeLU(XA)B, Megatron-LM tensor-parallel
// explainer, section 2.1):
//   forward   [QKV | FC1]:  a [T,h]      x [W_qkv | W_fc1]      -> qkv, u, GeLU(u)
//             [O ; FC2]:    [c | g]      x [W_o ; W_fc2]  + x   -> y
//   backward  dgrad:        dy x [W_o ; W_fc2]^T  (x GeLU'(u))  -> dc, du
//                           dZ x [W_qkv | W_fc1]^T              -> da (fp32)
//             wgrad:        [c | g]^T x dy                      -> dW_o, dW_fc2
//                           a^T x dZ                            -> dW_qkv, dW_fc1
// Concatenations are addressed in place (two-segment operands), never copied.
//
// Tiling: a 256-thread workgroup (4 waves of 64 lanes, 2 x 2) owns a BM x BN
// tile of C and walks K in steps of 64.  Both operands are staged in LDS as
// rows of 64 k-values (128 bytes, XOR-swizzled) so that every MFMA fragment is
// one 16-byte LDS read.  An operand whose k index is not contiguous in memory
// (weights in the forward, activations in the weight gradients) is loaded
// 16 bytes at a time along its contiguous dimension and transposed in
// registers on the way into LDS.  The next K tile is fetched into registers
// while the current one feeds the matrix cores.  Tiles are handed out
// XCD-aware: consecutive workgroups go round-robin over the 8 XCDs, so the
// tile index is remapped to give each XCD a contiguous, L2-friendly group of
// tiles.
#include "device_common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int BK = 64;

__device__ __forceinline__ const u16* operand_ptr(const Operand& op, int r, int k,
                                                  bool kmajor) {
  const u16* base = op.p0;
  int ld = op.ld0;
  if (op.split_on_k) {
    if (k >= op.split) { base = op.p1; ld = op.ld1; k -= op.split; }
  } else {
    if (r >= op.split) { base = op.p1; ld = op.ld1; r -= op.split; }
  }
  return kmajor ? base + (r * ld + k) : base + (k * ld + r);
}

template <int R, int MAJ>
struct TileLoader;

// k contiguous in memory: 16-byte chunks go straight to LDS.
template <int R>
struct TileLoader<R, KMAJOR> {
  static constexpr int NCH = R / 32;
  uint4 v[NCH];

  __device__ __forceinline__ void load(const Operand& op, int r0, int k0, int rlim,
                                       int K, int tid) {
    const int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = r0 + rr + 32 * i, k = k0 + c * 8;
      if (r < rlim && k < K)
        v[i] = *reinterpret_cast<const uint4*>(operand_ptr(op, r, k, true));
      else
        v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(u16* lds, int tid) const {
    const int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int r = rr + 32 * i;
      *reinterpret_cast<uint4*>(lds + r * BK + ((c ^ swz128(r)) << 3)) = v[i];
    }
  }
};

// Outer index contiguous in memory: each thread loads a KS x 8 block
// (KS k-rows of 8 consecutive outer indices) and writes it transposed.
template <int R>
struct TileLoader<R, OUTER_MAJOR> {
  static constexpr int RG = R / 8;
  static constexpr int KS = BK * RG / 256;  // 8 for R = 256, 4 for R = 128
  uint32_t w[KS][4];

  __device__ __forceinline__ void load(const Operand& op, int r0, int k0, int rlim,
                                       int K, int tid) {
    const int rg = tid % RG, kg = tid / RG;
    const int r = r0 + rg * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k = k0 + kg * KS + kk;
      uint4 t = make_uint4(0u, 0u, 0u, 0u);
      if (r < rlim && k < K) t = *reinterpret_cast<const uint4*>(operand_ptr(op, r, k, false));
      w[kk][0] = t.x; w[kk][1] = t.y; w[kk][2] = t.z; w[kk][3] = t.w;
    }
  }
  __device__ __forceinline__ void store(u16* lds, int tid) const {
    const int rg = tid % RG, kg = tid / RG;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = rg * 8 + j;
      uint32_t o[KS / 2];
#pragma unroll
      for (int p = 0; p < KS / 2; ++p) {
        const uint32_t a = w[2 * p][j >> 1], b = w[2 * p + 1][j >> 1];
        o[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      if constexpr (KS == 8) {
        *reinterpret_cast<uint4*>(lds + row * BK + ((kg ^ swz128(row)) << 3)) =
            make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        *reinterpret_cast<uint2*>(lds + row * BK + (((kg >> 1) ^ swz128(row)) << 3) +
                                  ((kg & 1) << 2)) = make_uint2(o[0], o[1]);
      }
    }
  }
};

__device__ __forceinline__ bf16x8 frag(const u16* lds, int row, int chunk) {
  return as_bf16x8(
      *reinterpret_cast<const uint4*>(lds + row * BK + ((chunk ^ swz128(row)) << 3)));
}

template <int MODE>
__device__ __forceinline__ void epi_apply(const Epilogue& e, int r, int c, float v) {
  if constexpr (MODE == EPI_QKV_GELU) {
    if (c < e.split) {
      e.o0[r * e.ld0 + c] = f2bf(v);
    } else {
      const int cc = c - e.split;
      e.o1[r * e.ld1 + cc] = f2bf(v);
      e.o2[r * e.ld1 + cc] = f2bf(gelu_f(v));
    }
  } else if constexpr (MODE == EPI_RESIDUAL) {
    e.o0[r * e.ld0 + c] = f2bf(v + bf2f(e.i0[r * e.ld0 + c]));
  } else if constexpr (MODE == EPI_DGELU) {
    if (c < e.split) {
      e.o0[r * e.ld0 + c] = f2bf(v);
    } else {
      const int cc = c - e.split;
      e.o1[r * e.ld1 + e.col_off1 + cc] = f2bf(v * gelu_grad_f(bf2f(e.i0[r * e.ld2 + cc])));
    }
  } else if constexpr (MODE == EPI_STORE2_COLS) {
    if (c < e.split) e.o0[r * e.ld0 + c] = f2bf(v);
    else e.o1[r * e.ld1 + (c - e.split)] = f2bf(v);
  } else if constexpr (MODE == EPI_STORE2_ROWS) {
    if (r < e.split) e.o0[r * e.ld0 + c] = f2bf(v);
    else e.o1[(r - e.split) * e.ld1 + c] = f2bf(v);
  } else {
    e.of[r * e.ld0 + c] = v;
  }
}

template <int BM, int BN, int AMAJ, int BMAJ, int MODE>
__global__ __launch_bounds__(256, 1) void gemm_kernel(int M, int N, int K, Operand A,
                                                      Operand B, Epilogue epi) {
  constexpr int WM = BM / 2, WN = BN / 2;  // per-wave tile
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int STAGE = (BM + BN) * BK;
  __shared__ __attribute__((aligned(16))) u16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile index: XCD-aware remap, then grouped row-major order
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int nt = tiles_m * tiles_n;
  int pid = blockIdx.x;
  {
    const int per = (nt + 7) / 8;
    const int tall = (nt % 8 == 0) ? 8 : nt % 8;
    const int xcd = pid % 8, loc = pid / 8;
    pid = xcd < tall ? xcd * per + loc : tall * per + (xcd - tall) * (per - 1) + loc;
  }
  constexpr int GM = 8;
  const int span = GM * tiles_n;
  const int first_m = (pid / span) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % span) % gsz;
  const int tn = (pid % span) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  TileLoader<BM, AMAJ> la;
  TileLoader<BN, BMAJ> lb;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  la.load(A, m0, 0, M, K, tid);
  lb.load(B, n0, 0, N, K, tid);
  la.store(smem, tid);
  lb.store(smem + BM * BK, tid);
  __syncthreads();

  const int lrow = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, m0, (kt + 1) * BK, M, K, tid);
      lb.load(B, n0, (kt + 1) * BK, N, K, tid);
    }
    const u16* As = smem + cur * STAGE;
    const u16* Bs = As + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = frag(As, wm * WM + i * 32 + lrow, ks * 2 + lk);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = frag(Bs, wn * WN + j * 32 + lrow, ks * 2 + lk);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      u16* nxt = smem + (cur ^ 1) * STAGE;
      la.store(nxt, tid);
      lb.store(nxt + BM * BK, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds C[row0 + 8*jj + 4*lk + ii][col]
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + lrow;
      if (col >= N) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int row = m0 + wm * WM + i * 32 + jj * 8 + lk * 4 + ii;
          if (row < M) epi_apply<MODE>(epi, row, col, acc[i][j][jj * 4 + ii]);
        }
      }
    }
  }
}

template <int BM, int BN, int AMAJ, int BMAJ, int MODE>
hipError_t launch_tiles(int M, int N, int K, const Operand& A, const Operand& B,
                        const Epilogue& e, hipStream_t s) {
  const int nt = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AMAJ, BMAJ, MODE>), dim3(nt), dim3(256), 0, s,
                     M, N, K, A, B, e);
  return hipGetLastError();
}

template <int AMAJ, int BMAJ, int MODE>
hipError_t launch_sized(int M, int N, int K, const Operand& A, const Operand& B,
                        const Epilogue& e, hipStream_t s) {
  const long big = static_cast<long>((M + 255) / 256) * ((N + 255) / 256);
  if (big >= 192) return launch_tiles<256, 256, AMAJ, BMAJ, MODE>(M, N, K, A, B, e, s);
  return launch_tiles<128, 128, AMAJ, BMAJ, MODE>(M, N, K, A, B, e, s);
}

}  // namespace

hipError_t launch_gemm(int M, int N, int K, const Operand& A, Major a_major,
                       const Operand& B, Major b_major, EpiMode mode,
                       const Epilogue& e, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  // The combinations used by the layer; anything else is a library bug.
  if (a_major == KMAJOR && b_major == OUTER_MAJOR) {
    if (mode == EPI_QKV_GELU) return launch_sized<KMAJOR, OUTER_MAJOR, EPI_QKV_GELU>(M, N, K, A, B, e, s);
    if (mode == EPI_RESIDUAL) return launch_sized<KMAJOR, OUTER_MAJOR, EPI_RESIDUAL>(M, N, K, A, B, e, s);
  } else if (a_major == KMAJOR && b_major == KMAJOR) {
    if (mode == EPI_DGELU) return launch_sized<KMAJOR, KMAJOR, EPI_DGELU>(M, N, K, A, B, e, s);
    if (mode == EPI_F32) return launch_sized<KMAJOR, KMAJOR, EPI_F32>(M, N, K, A, B, e, s);
  } else if (a_major == OUTER_MAJOR && b_major == OUTER_MAJOR) {
    if (mode == EPI_STORE2_ROWS) return launch_sized<OUTER_MAJOR, OUTER_MAJOR, EPI_STORE2_ROWS>(M, N, K, A, B, e, s);
    if (mode == EPI_STORE2_COLS) return launch_sized<OUTER_MAJOR, OUTER_MAJOR, EPI_STORE2_COLS>(M, N, K, A, B, e, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ptb
