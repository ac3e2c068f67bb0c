// Host-side launchers of the gfx950 kernels (internal to libptb).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptb {

typedef uint16_t u16;

// A GEMM operand made of up to two row-major bf16 segments that together form
// one logical matrix.  `split` is where segment 1 starts along the split
// dimension: the contraction index k (split_on_k = 1) or the outer index (the
// output row for A, the output column for B; split_on_k = 0).  Indices inside
// segment 1 are taken relative to `split`.  This addresses the concatenated
// weights [W_qkv | W_fc1] and [W_o ; W_fc2] and the concatenated activations
// [c | g] in place, without copying them.
// bytes0/bytes1 bound each segment: reads at or past them return zero.  Split
// points must be multiples of 64.
struct Operand {
  const u16* p0;
  const u16* p1;
  int ld0;
  int ld1;
  int split;
  int split_on_k;
  uint32_t bytes0;
  uint32_t bytes1;
};

// Storage order of an operand: KMAJOR means element (outer r, k) sits at
// r*ld + k (k contiguous); OUTER_MAJOR means it sits at k*ld + r.
enum Major { KMAJOR = 0, OUTER_MAJOR = 1 };

// What the GEMM does with each fp32 result v at (row r, column c).
enum EpiMode {
  EPI_QKV_GELU = 0,  // with gc = c + col_base: gc < split: o0[r*ld0+gc] = bf16(v), and
                     // for gc < lo_cols also o3[r*ld3+gc] = fp16(v) (saturated);
                     // else o1 = v (u), o2 = GeLU(v) (g) at column gc - split
  EPI_RESIDUAL = 1,  // o0[r*ld0+c] = D(v) + i0[r*ld0+c], D the dropout `drop` of element
                     // r*ld0+c (the identity when drop.on = 0; FP8 products ignore
                     // `drop`: FP8 layers take no dropout)
  EPI_DGELU = 2,     // c < split: o0[r*ld0+c] = v; else o1[r*ld1+col_off1+c-split] =
                     //   v * GeLU'(i0[r*ld2 + c-split])
  EPI_STORE2_COLS = 3,  // c < split: o0[r*ld0+c]; else o1[r*ld1 + c-split]
  EPI_STORE2_ROWS = 4,  // r < split: o0[r*ld0+c]; else o1[(r-split)*ld1 + c]
  EPI_F32 = 5,          // of[r*ld0+c] = v (fp32)
  EPI_QKV_SWIGLU = 6,   // as EPI_QKV_GELU below `split`; at and above it the columns
                        // are SwiGLU's [W1 | W3] in 32-wide blocks alternating W1, W3:
                        // with cc = gc - split, the pair of blocks at cc = 64 j (W1)
                        // and 64 j + 32 (W3) is stored as is to o1 (ld1) and
                        // g = silu(u1) * u3 to o2[r*ld2 + 32 j ..] (eight-wave
                        // kernel: a wave's two 32-column blocks are such a pair)
  EPI_DSWIGLU = 7       // c < split: o0[r*ld0+c] = v; else, with cc = c - split in
                        // [32 j, 32 j + 32) and u1, u3 read from i0 (ld2) at
                        // columns 64 j + cc % 32 and + 32:
                        // o1[r*ld1 + col_off1 + 64 j + cc % 32] = v * u3 * silu'(u1),
                        // o1[... + 32] = v * silu(u1)
};

// Dropout of a [rows, ld] tensor (the block's branch output, before the
// residual add): element e = r * ld + c is kept iff word e & 3 of
// Philox-4x32-10 of the counter (e >> 2, stream, 0, 0) under the key
// (k0, k1) is >= t = floor(p 2^32), and a kept element is multiplied by
// scale = 1 / (1 - p).  on = 0 for p = 0 (nothing dropped or scaled).
struct Dropout {
  uint32_t k0, k1;    // key: the seed's low and high words
  uint32_t stream;    // 2 * layer (+ 1 for the serial block's MLP branch)
  uint32_t t;         // keep threshold
  float scale;
  int on;
};

struct Epilogue {
  u16* o0;
  u16* o1;
  u16* o2;
  u16* o3;
  float* of;
  const u16* i0;
  int ld0, ld1, ld2, ld3;
  int col_off1;
  int col_base;
  int lo_cols;
  int split;
  Dropout drop;  // EPI_RESIDUAL: dropout of the product before the residual add
};

// One matrix product C[M,N] = A[M,K] * B[K,N] and what happens to C.
struct GemmProblem {
  int M, N, K;
  Operand A, B;
  Epilogue epi;
};

// The two 8-bit float formats (Megatron-LM tuning post, mixed precision):
// E4M3 (largest 448) and E5M2 (largest 57344), OCP encodings.
enum Fp8Format { FP8_E4M3 = 0, FP8_E5M2 = 1 };

// Block-scaled (MX) FP8: blocks of 32 consecutive values along a copy's
// contiguous (contraction) dimension, one E8M0 scale each (code e means
// 2^(e - 127)).  A copy's scales are ld bytes x 4 per 128-wide k-step ks
// (ld >= rows, a multiple of 128), in the order the matrix cores' lanes take
// them: for row r = 128 g + 32 i + l (i < 4, l < 32), the code of k-block
// 4 ks + b sits at byte mx_scale_byte(ks, r, b, ld) = 4 (ks ld + 128 g) +
// 16 l + 8 (b & 1) + 4 (b >> 1) + i.  A wave holding rows 128 g + 32 i + l
// (fragment i of lane l and l + 32) then finds in the 8 bytes at
// 16 l + 8 h' of the group the codes lane half h' supplies for both
// 64-wide halves of the k-step, one byte per fragment.
constexpr size_t mx_scale_byte(int ks, int r, int b, int ld) {
  return 4 * (static_cast<size_t>(ks) * ld + (r & ~127)) + 16 * (r & 31) + 8 * (b & 1) +
         4 * (b >> 1) + ((r >> 5) & 3);
}
struct MxScales {
  const uint32_t* p;
  int ld;
};

// Scratch of the GEMM launches: fp32 partial sums of 256 x 256 tiles that
// are split along k (kGemmPartialSlots of them at most) and one arrival
// counter per output tile.  The counters must be zero before a launch; every
// launch leaves them zero, so launches on one stream can share them.
constexpr int kGemmMaxWorkgroups = 256;
constexpr int kGemmPartialSlots = 1024;
constexpr size_t kGemmPartialBytes =
    static_cast<size_t>(kGemmPartialSlots) * 256 * 256 * sizeof(float);
struct GemmScratch {
  float* partials;  // kGemmPartialBytes
  int* counters;    // max_tiles ints
  int max_tiles;
};

// Output tiles of an M x N product (the counters one launch needs).
int gemm_tiles(int M, int N);

// p[0 .. n) = 0 (clears the counters at the start of a layer call).
hipError_t launch_zero_i32(int* p, int n, hipStream_t stream);

// C[M,N] = A[M,K] * B[K,N] with the epilogue applied to C.  Operands must be
// 16-byte aligned with leading dimensions that are multiples of 8; K must be
// a multiple of 32 when either operand is k-contiguous.
hipError_t launch_gemm(int M, int N, int K, const Operand& A, Major a_major,
                       const Operand& B, Major b_major, EpiMode mode,
                       const Epilogue& epi, const GemmScratch& scratch, hipStream_t stream);

// Up to two independent products sharing operand orders and epilogue kind,
// in one launch (the tiles of both fill the GPU together).  f16_prob0:
// problem 0's operands hold fp16 values instead of bf16 (the [q | k]
// product of the [QKV | FC1] launch; KMAJOR x OUTER_MAJOR, EPI_QKV_* only).
hipError_t launch_gemm_group(const GemmProblem* probs, int nprob, Major a_major,
                             Major b_major, EpiMode mode, const GemmScratch& scratch,
                             hipStream_t stream, bool f16_prob0 = false);

// FP8 product: both operands k-contiguous 8-bit matrices (element (r, k) at
// byte r*ld + k, ld a multiple of 16), K a multiple of 128, fa / fb their
// formats and amax_a / amax_b their amax (device memory, written by
// launch_amax): the epilogue sees C / (sA sB) with sX = FMAX_X / amax_X.  The modes the FP8 layer uses: EPI_QKV_GELU and EPI_RESIDUAL
// (E4M3 x E4M3), EPI_DGELU and EPI_STORE2_COLS (E5M2 x E4M3),
// EPI_STORE2_ROWS and EPI_STORE2_COLS (E4M3 x E5M2).
hipError_t launch_gemm_fp8(const GemmProblem& prob, Fp8Format fa, const float* amax_a,
                           Fp8Format fb, const float* amax_b, EpiMode mode,
                           const GemmScratch& scratch, hipStream_t stream);

// The same products on block-scaled (MX) operands: the scales are applied by
// the matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), so the epilogue sees C
// itself.  sa holds the scale words of A's M rows, sb those of B's N rows
// (B stored k-contiguous, [N][K]), K a multiple of 128.
hipError_t launch_gemm_mx(const GemmProblem& prob, Fp8Format fa, const MxScales& sa,
                          Fp8Format fb, const MxScales& sb, EpiMode mode,
                          const GemmScratch& scratch, hipStream_t stream);

// A logical bf16 matrix X [R, C] made of up to two row-major segments:
// columns [0, split) from p0 (ld0) and [split, C) from p1 (ld1) when
// split_on_rows = 0, rows likewise when it is 1 (split >= C or R: one
// segment).  Leading dimensions and split are multiples of 8.
struct CastSrc {
  const u16* p0;
  const u16* p1;
  int ld0, ld1;
  int split, split_on_rows;
  int R, C;
};

// *amax = max(*amax, max |X|) (as float bits; *amax starts at 0).  Each
// segment must be a plain array (its leading dimension equal to its width).
hipError_t launch_amax(const CastSrc& x, float* amax, hipStream_t stream);

// FP8 copies of X on its current scale s = FMAX / *amax: rows[r*ldr + c]
// (ldr >= C) and/or cols[c*ldc + r] (the transpose, ldc >= R), each code
// round-to-nearest-even of clamp(x * s) with x * s in fp32; padding columns
// (c in [C, ldr) of rows, r in [R, ldc) of cols) are written as zero.
// ldr and ldc are multiples of 64; either output may be null.
hipError_t launch_cast_fp8(const CastSrc& x, Fp8Format fmt, const float* amax, uint8_t* rows,
                           int ldr, uint8_t* cols, int ldc, hipStream_t stream);

// Block-scaled FP8 copies of X: code = RNE(clamp(x 2^-X, -FMAX, FMAX)) with
// X = floor(log2 amax_block) - emax (emax 8 for E4M3, 15 for E5M2; 0 for an
// all-zero block), written row-wise to rows [R][ldr] with scales rs
// (MxScales layout, ld rs_ld >= R) and/or transposed to cols [C][ldc] with
// scales cs (ld cs_ld >= C).  ldr and ldc are multiples of 128 (whole
// k-steps); padding codes are zero, padding blocks and rows get code 127.
hipError_t launch_cast_mx(const CastSrc& x, Fp8Format fmt, uint8_t* rows, int ldr, uint32_t* rs,
                          int rs_ld, uint8_t* cols, int ldc, uint32_t* cs, int cs_ld,
                          hipStream_t stream);

// dst[e] = D(src[e]) for e < n (n a multiple of 8, 16-byte aligned bf16
// arrays): the dropout of the backward's upstream gradient of a branch.
hipError_t launch_dropout_apply(const u16* src, u16* dst, long n, const Dropout& d,
                                hipStream_t stream);
// mask[e] = 1 if element e is kept, else 0, for e < n (bytes).
hipError_t launch_dropout_mask(uint8_t* mask, long n, const Dropout& d, hipStream_t stream);

// LayerNorm forward over rows of x [T, h]: a = bf16(LN(x)) and an fp16 copy
// a16 = fp16(LN(x)) of the same fp32 values (skipped when a16 is null), mu,
// rstd (fp32).  rms: RMSNorm instead (no mean, no beta; mu is written as 0).
// clear[0, nclear), if given, is set to zero by the same launch.
hipError_t launch_layernorm_fwd(const u16* x, const u16* gamma, const u16* beta,
                                u16* a, u16* a16, float* mu, float* rstd, int T, int h,
                                float eps, hipStream_t stream, bool rms = false,
                                int* clear = nullptr, int nclear = 0);

// dst = fp16(src) for a [rows, cols] block of a row-major bf16 matrix (cols
// and both row strides multiples of 8; rounding to nearest even, saturated
// at 65504).
hipError_t launch_cast_f16(const u16* src, int ld_src, int rows, int cols, u16* dst, int ld_dst,
                           hipStream_t stream);

// LayerNorm backward plus residual: dx = dy + LN'(da); per-block partial sums
// of dgamma, dbeta into `partials` [nblk, 2, h], then reduced into bf16.
int layernorm_bwd_blocks(int T);
hipError_t launch_layernorm_bwd(const u16* da, const u16* x, const u16* gamma,
                                const float* mu, const float* rstd, const u16* dy,
                                u16* dx, float* partials, u16* dgamma, u16* dbeta,
                                int T, int h, hipStream_t stream, bool rms = false);

// Scratch of the attention launches: fp32 partial results of rows split into
// chunks, and one arrival counter per (batch, head, row) (zero on entry, left
// zero).  cus = compute units of the device (sets the chunking).
struct AttnScratch {
  float* partials;
  size_t partial_floats;
  int* counters;
  int max_counters;
  int cus;
};

// Compute units of the current device (0 if the query fails).
int device_compute_units();

// Sliding-window causal flash attention, forward: reads the bf16 v column
// block of qkv [b*s, 3*n*d] and the fp16 q and k of qk16 [b*s, 2*n*d]
// (logits from one fp16 product); writes c [b*s, n*d] and the base-2
// log-sum-exp lse [b, n, s].
hipError_t launch_attention_fwd(const u16* qkv, const u16* qk16, u16* c, float* lse,
                                int b, int s, int n, int d, int window,
                                const AttnScratch& scratch, hipStream_t stream);

// Attention backward.  delta[b,n,s] = rowsum(dc * c) per head first, then
// dk, dv and dq written into the first 3*n*d columns of dz [b*s, ld_dz].
// q and k are read from qk16 (fp16), v from qkv (bf16).
hipError_t launch_attention_bwd(const u16* qkv, const u16* qk16, const u16* c,
                                const float* lse, const u16* dc, float* delta, u16* dz,
                                int ld_dz, int b, int s, int n, int d, int window,
                                const AttnScratch& scratch, hipStream_t stream);

// LAMB step over up to kLambMaxTensors parameter tensors (each its own
// "layer" for the trust ratio): fp32 master weights theta and moments m, v
// updated in place from the bf16 gradient, and the bf16 copy of theta written
// to `weight`.  numel must be a multiple of 8 and every pointer 16-byte
// aligned.  `partial` holds 2 doubles per workgroup (sum of lamb_blocks over
// the tensors), `norms` 2 floats per tensor (||theta||, ||r|| of this step).
constexpr int kLambMaxTensors = 32;
struct LambTensor {
  float* theta;
  float* m;
  float* v;
  const u16* grad;
  u16* weight;
  long numel;
};
struct LambHyper {
  float lr, beta1, beta2, eps;
  int step;
};
int lamb_blocks(long numel);
// The allocation-free step's scratch: a static device array of this many
// bytes (room for the partial sums of this many / 16 workgroups), one per
// GPU.  lamb_static_scratch returns its address on the current device,
// looked up once per device.
constexpr size_t kLambStaticScratchBytes = size_t(4) << 20;
hipError_t lamb_static_scratch(double** out);
hipError_t launch_lamb(const LambTensor* ts, int n, const LambHyper& hp, double* partial,
                       float* norms, hipStream_t stream);

}  // namespace ptb
