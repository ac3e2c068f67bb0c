// Host-only stand-ins for libptb's kernel launchers, for a sanitizer build of
// the C ABI's host code (ptb_api.cpp) without a GPU.  Each stand-in touches
// the first and the last byte of every buffer region the API hands to a
// kernel, as the kernel's extent arguments describe it; the driver passes
// real host allocations sized by the library's own size queries, so a wrong
// offset or extent in the saved/workspace layouts or the launch arguments
// becomes an AddressSanitizer report.  Nothing is computed.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "../../transformer_block_amd/csrc/kernels.h"

namespace {
volatile unsigned char g_sink;

void touch(const void* p, size_t bytes) {
  if (p == nullptr || bytes == 0) return;
  const volatile unsigned char* b = static_cast<const volatile unsigned char*>(p);
  g_sink = g_sink ^ b[0] ^ b[bytes - 1];
}
// element (row, col) of a row-major matrix of `esz`-byte elements: touch its
// byte range
void touch_at(const void* p, long row, long ld, long col, size_t esz) {
  if (p == nullptr || row < 0 || col < 0) return;
  const unsigned char* b = static_cast<const unsigned char*>(p);
  touch(b + (row * ld + col) * static_cast<long>(esz), esz);
}
void touch_matrix(const void* p, long rows, long ld, long cols, size_t esz) {
  if (rows <= 0 || cols <= 0) return;
  touch_at(p, 0, ld, 0, esz);
  touch_at(p, rows - 1, ld, cols - 1, esz);
}
void touch_operand(const ptb::Operand& op) {
  touch(op.p0, op.bytes0);
  touch(op.p1, op.bytes1);
}
long pad128(long v) { return (v + 127) / 128 * 128; }

void touch_epilogue(const ptb::GemmProblem& p, ptb::EpiMode mode) {
  const ptb::Epilogue& e = p.epi;
  const long M = p.M, N = p.N;
  switch (mode) {
    case ptb::EPI_QKV_GELU:
    case ptb::EPI_QKV_SWIGLU: {
      // global columns [col_base, col_base + N): below split -> o0 (and o3
      // below lo_cols), at and above it -> o1 (u) and o2 (g)
      const long g0 = e.col_base, g1 = e.col_base + N;
      if (g0 < e.split) touch_matrix(e.o0, M, e.ld0, std::min<long>(g1, e.split), 2);
      if (g0 < e.lo_cols) touch_matrix(e.o3, M, e.ld3, std::min<long>(g1, e.lo_cols), 2);
      if (g1 > e.split) {  // FC1-side columns up to g1 - split of u (and of g)
        const long cc = g1 - e.split;
        touch_matrix(e.o1, M, e.ld1, cc, 2);
        touch_matrix(e.o2, M, e.ld2, mode == ptb::EPI_QKV_SWIGLU ? cc / 2 : cc, 2);
      }
      break;
    }
    case ptb::EPI_RESIDUAL:
      touch_matrix(e.o0, M, e.ld0, N, 2);
      touch_matrix(e.i0, M, e.ld0, N, 2);
      break;
    case ptb::EPI_DGELU:
    case ptb::EPI_DSWIGLU:
      touch_matrix(e.o0, M, e.ld0, std::min<long>(N, e.split), 2);
      if (N > e.split) {
        touch_matrix(e.o1, M, e.ld1, e.col_off1 + (mode == ptb::EPI_DSWIGLU ? 2 : 1) * (N - e.split), 2);
        touch_matrix(e.i0, M, e.ld2, (mode == ptb::EPI_DSWIGLU ? 2 : 1) * (N - e.split), 2);
      }
      break;
    case ptb::EPI_STORE2_COLS:
      touch_matrix(e.o0, M, e.ld0, std::min<long>(N, e.split), 2);
      if (N > e.split) touch_matrix(e.o1, M, e.ld1, N - e.split, 2);
      break;
    case ptb::EPI_STORE2_ROWS:
      touch_matrix(e.o0, std::min<long>(M, e.split), e.ld0, N, 2);
      if (M > e.split) touch_matrix(e.o1, M - e.split, e.ld1, N, 2);
      break;
    case ptb::EPI_F32:
      touch_matrix(e.of, M, e.ld0, N, 4);
      break;
  }
}
void touch_scratch(const ptb::GemmScratch& s) {
  touch(s.partials, ptb::kGemmPartialBytes);
  touch(s.counters, static_cast<size_t>(s.max_tiles) * 4);
}
void touch_cast_src(const ptb::CastSrc& x) {
  if (x.split_on_rows) {
    touch_matrix(x.p0, std::min(x.split, x.R), x.ld0, x.C, 2);
    if (x.R > x.split) touch_matrix(x.p1, x.R - x.split, x.ld1, x.C, 2);
  } else {
    touch_matrix(x.p0, x.R, x.ld0, std::min(x.split, x.C), 2);
    if (x.C > x.split) touch_matrix(x.p1, x.R, x.ld1, x.C - x.split, 2);
  }
}
alignas(256) unsigned char g_lamb_scratch[ptb::kLambStaticScratchBytes];
}  // namespace

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace ptb {

// the library's tile count (256 x 256 output tiles), as in gemm.hip
int gemm_tiles(int M, int N) { return ((M + 255) / 256) * ((N + 255) / 256); }
int device_compute_units() { return 256; }
int layernorm_bwd_blocks(int T) { return T < 256 ? (T < 1 ? 1 : T) : 256; }
int lamb_blocks(long numel) { return static_cast<int>((numel + 16383) / 16384); }

hipError_t launch_zero_i32(int* p, int n, hipStream_t) {
  touch(p, static_cast<size_t>(n) * 4);
  return hipSuccess;
}

hipError_t launch_gemm_group(const GemmProblem* probs, int nprob, Major, Major, EpiMode mode,
                             const GemmScratch& s, hipStream_t, bool) {
  for (int i = 0; i < nprob; ++i) {
    touch_operand(probs[i].A);
    touch_operand(probs[i].B);
    touch_epilogue(probs[i], mode);
  }
  touch_scratch(s);
  return hipSuccess;
}

hipError_t launch_gemm(int M, int N, int K, const Operand& A, Major am, const Operand& B,
                       Major bm, EpiMode mode, const Epilogue& epi, const GemmScratch& s,
                       hipStream_t st) {
  GemmProblem p{M, N, K, A, B, epi};
  return launch_gemm_group(&p, 1, am, bm, mode, s, st, false);
}

hipError_t launch_gemm_fp8(const GemmProblem& p, Fp8Format, const float* amax_a, Fp8Format,
                           const float* amax_b, EpiMode mode, const GemmScratch& s, hipStream_t) {
  touch_operand(p.A);
  touch_operand(p.B);
  touch_epilogue(p, mode);
  touch(amax_a, 4);
  touch(amax_b, 4);
  touch_scratch(s);
  return hipSuccess;
}

hipError_t launch_gemm_mx(const GemmProblem& p, Fp8Format, const MxScales& sa, Fp8Format,
                          const MxScales& sb, EpiMode mode, const GemmScratch& s, hipStream_t) {
  touch_operand(p.A);
  touch_operand(p.B);
  touch_epilogue(p, mode);
  const long ks = pad128(p.K) / 128;
  // the kernel reads the scales of whole 256-row tiles, bounded by the array
  touch_matrix(sa.p, ks, sa.ld, sa.ld, 4);
  touch_matrix(sb.p, ks, sb.ld, sb.ld, 4);
  touch_scratch(s);
  return hipSuccess;
}

hipError_t launch_amax(const CastSrc& x, float* amax, hipStream_t) {
  touch_cast_src(x);
  touch(amax, 4);
  return hipSuccess;
}

hipError_t launch_cast_fp8(const CastSrc& x, Fp8Format, const float* amax, uint8_t* rows, int ldr,
                           uint8_t* cols, int ldc, hipStream_t) {
  touch_cast_src(x);
  touch(amax, 4);
  if (rows) touch_matrix(rows, x.R, ldr, ldr, 1);
  if (cols) touch_matrix(cols, x.C, ldc, ldc, 1);
  return hipSuccess;
}

hipError_t launch_cast_mx(const CastSrc& x, Fp8Format, uint8_t* rows, int ldr, uint32_t* rs,
                          int rs_ld, uint8_t* cols, int ldc, uint32_t* cs, int cs_ld,
                          hipStream_t) {
  touch_cast_src(x);
  if (rows) {
    touch_matrix(rows, x.R, ldr, ldr, 1);
    touch_matrix(rs, ldr / 128, rs_ld, rs_ld, 4);
  }
  if (cols) {
    touch_matrix(cols, x.C, ldc, ldc, 1);
    touch_matrix(cs, ldc / 128, cs_ld, cs_ld, 4);
  }
  return hipSuccess;
}

hipError_t launch_dropout_apply(const u16* src, u16* dst, long n, const Dropout&, hipStream_t) {
  touch(src, n * 2);
  touch(dst, n * 2);
  return hipSuccess;
}

hipError_t launch_dropout_mask(uint8_t* mask, long n, const Dropout&, hipStream_t) {
  touch(mask, n);
  return hipSuccess;
}

hipError_t launch_layernorm_fwd(const u16* x, const u16* gamma, const u16* beta, u16* a, u16* a16,
                                float* mu, float* rstd, int T, int h, float, hipStream_t, bool,
                                int* clear, int nclear) {
  touch(clear, static_cast<size_t>(nclear > 0 ? nclear : 0) * 4);
  touch(x, static_cast<size_t>(T) * h * 2);
  touch(a, static_cast<size_t>(T) * h * 2);
  touch(a16, static_cast<size_t>(T) * h * 2);
  touch(gamma, h * 2);
  touch(beta, h * 2);
  touch(mu, T * 4);
  touch(rstd, T * 4);
  return hipSuccess;
}

hipError_t launch_cast_f16(const u16* src, int ld_src, int rows, int cols, u16* dst, int ld_dst,
                           hipStream_t) {
  touch_matrix(src, rows, ld_src, cols, 2);
  touch_matrix(dst, rows, ld_dst, cols, 2);
  return hipSuccess;
}

hipError_t launch_layernorm_bwd(const u16* da, const u16* x, const u16* gamma, const float* mu,
                                const float* rstd, const u16* dy, u16* dx, float* partials,
                                u16* dgamma, u16* dbeta, int T, int h, hipStream_t, bool) {
  const size_t th = static_cast<size_t>(T) * h * 2;
  touch(da, th);
  touch(x, th);
  touch(dy, th);
  touch(dx, th);
  touch(gamma, h * 2);
  touch(mu, T * 4);
  touch(rstd, T * 4);
  touch(partials, static_cast<size_t>(layernorm_bwd_blocks(T)) * 2 * h * 4);
  touch(dgamma, h * 2);
  touch(dbeta, h * 2);
  return hipSuccess;
}

hipError_t launch_attention_fwd(const u16* qkv, const u16* qk16, u16* c, float* lse, int b, int s,
                                int n, int d, int, const AttnScratch& sc, hipStream_t) {
  const long T = static_cast<long>(b) * s, hl = static_cast<long>(n) * d;
  touch(qkv, T * 3 * hl * 2);
  touch(qk16, T * 2 * hl * 2);
  touch(c, T * hl * 2);
  touch(lse, static_cast<size_t>(b) * n * s * 4);
  touch(sc.partials, sc.partial_floats * 4);
  touch(sc.counters, static_cast<size_t>(sc.max_counters) * 4);
  return hipSuccess;
}

hipError_t launch_attention_bwd(const u16* qkv, const u16* qk16, const u16* c, const float* lse,
                                const u16* dc, float* delta, u16* dz, int ld_dz, int b, int s,
                                int n, int d, int, const AttnScratch& sc, hipStream_t) {
  const long T = static_cast<long>(b) * s, hl = static_cast<long>(n) * d;
  touch(qkv, T * 3 * hl * 2);
  touch(qk16, T * 2 * hl * 2);
  touch(c, T * hl * 2);
  touch(dc, T * hl * 2);
  touch(lse, static_cast<size_t>(b) * n * s * 4);
  touch(delta, static_cast<size_t>(b) * n * s * 4);
  touch_matrix(dz, T, ld_dz, 3 * hl, 2);
  touch(sc.partials, sc.partial_floats * 4);
  touch(sc.counters, static_cast<size_t>(sc.max_counters) * 4);
  return hipSuccess;
}

hipError_t lamb_static_scratch(double** out) {
  *out = reinterpret_cast<double*>(g_lamb_scratch);
  return hipSuccess;
}

hipError_t launch_lamb(const LambTensor* ts, int n, const LambHyper&, double* partial,
                       float* norms, hipStream_t) {
  long blocks = 0;
  for (int i = 0; i < n; ++i) {
    touch(ts[i].theta, ts[i].numel * 4);
    touch(ts[i].m, ts[i].numel * 4);
    touch(ts[i].v, ts[i].numel * 4);
    touch(ts[i].grad, ts[i].numel * 2);
    touch(ts[i].weight, ts[i].numel * 2);
    blocks += lamb_blocks(ts[i].numel);
  }
  touch(partial, blocks * 16);
  touch(norms, static_cast<size_t>(n) * 8);
  return hipSuccess;
}

}  // namespace ptb
