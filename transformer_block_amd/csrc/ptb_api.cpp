// C ABI of libptb (declared in include/ptb.h): argument checks, the layout of
// the forward->backward stash and of the backward scratch, and the launch
// sequence of one Parallel Transformer Block layer
//   y = x + Attn(LN(x)) + MLP(LN(x))
// (MegaScale reading notes, section 1.1, eq (4)).
//
// Forward, five launches on the caller's stream:
//   LN(x) -> a (+ its fp16 copy a16);  the q, k columns of W_qkv -> fp16;
//   a x [W_qkv | W_fc1] -> qkv, u, g = GeLU(u) (the q, k columns as the fp16
//   product a16 x W_q|k, kept in bf16 and in fp16 for the logits);
//   sliding-window flash attention -> c, lse;  [c | g] x [W_o ; W_fc2] + x -> y.
// Backward:
//   dy x [W_o ; W_fc2]^T -> dc, du = dg * GeLU'(u);  attention backward
//   (probabilities recomputed from lse) -> dq, dk, dv;  [c | g]^T dy -> dW_o, dW_fc2;
//   dZ x [W_qkv | W_fc1]^T -> da;  a^T dZ -> dW_qkv, dW_fc1;
//   LayerNorm backward + dy -> dx, dgamma, dbeta.
// dZ = [dq | dk | dv | du] is one [T, 3*h_l + f] buffer, so the two products
// with [W_qkv | W_fc1] each run as a single GEMM.
//
// The serial block (same notes, eq (3), read with the attention residual:
// x1 = x + Attn(LN1(x)) W_o, y = x1 + MLP(LN2(x1))) runs the same kernels with
// the products separate: seven forward and eleven backward stages.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <initializer_list>

#include "../../include/ptb.h"
#include "kernels.h"

namespace {

using ptb::u16;

static_assert(PTB_LAMB_NOALLOC_SCRATCH_BYTES == ptb::kLambStaticScratchBytes,
              "the header's static scratch size is the library's");

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Shape {
  long b, s, h, n, d, f, w, T, hl, N1, K2;
  long f1;      // FC1 output width: f (GeLU) or 2f (SwiGLU's [W1 | W3])
  bool rms;     // RMSNorm instead of LayerNorm
  bool swiglu;  // SwiGLU MLP instead of GeLU
};

int32_t check_dims(const ptb_dims* dims, Shape* out) {
  if (dims == nullptr) return PTB_ERR_NULL;
  const ptb_dims& p = *dims;
  if (p.batch < 1 || p.seq < 1 || p.heads < 1) return PTB_ERR_DIMS;
  if (p.head_dim != 64 && p.head_dim != 128) return PTB_ERR_HEAD_DIM;
  if (p.hidden < 64 || p.hidden % 64 != 0 || p.hidden > 16384) return PTB_ERR_DIMS;
  if (p.ffn < 64 || p.ffn % 64 != 0) return PTB_ERR_DIMS;
  if (p.window < 1) return PTB_ERR_WINDOW;
  if (!(p.ln_eps > 0.0f) || !isfinite(p.ln_eps)) return PTB_ERR_EPS;
  if ((p.norm != PTB_NORM_LAYERNORM && p.norm != PTB_NORM_RMSNORM) ||
      (p.mlp != PTB_MLP_GELU && p.mlp != PTB_MLP_SWIGLU))
    return PTB_ERR_ARG;
  if (!(p.dropout_p >= 0.0f && p.dropout_p < 1.0f) || p.dropout_layer > 0x7fffffffu)
    return PTB_ERR_ARG;
  Shape s;
  s.b = p.batch; s.s = p.seq; s.h = p.hidden; s.n = p.heads; s.d = p.head_dim; s.f = p.ffn;
  s.w = p.window < p.seq ? p.window : p.seq;  // a window >= seq is full causal attention
  s.T = s.b * s.s;
  s.hl = s.n * s.d;
  s.rms = p.norm == PTB_NORM_RMSNORM;
  s.swiglu = p.mlp == PTB_MLP_SWIGLU;
  s.f1 = s.swiglu ? 2 * s.f : s.f;
  s.N1 = 3 * s.hl + s.f1;
  s.K2 = s.hl + s.f;
  const long lim = 1L << 30;
  // every tensor must stay below 2^31 bytes: kernels address it with 32-bit
  // byte offsets
  if (s.T > lim / s.N1 || s.h > lim / s.N1 || s.T > lim / s.h || s.K2 > lim / s.h ||
      s.b * s.n > lim / s.s)
    return PTB_ERR_DIMS;
  if (out) *out = s;
  return PTB_OK;
}

// The dropout of one branch output of the layer (MegaScale notes, section
// 1.3): stream 2 * layer + branch, threshold floor(p 2^32), scale 1 / (1 - p);
// off for p = 0.
ptb::Dropout dropout_of(const ptb_dims& p, uint32_t branch) {
  ptb::Dropout d{};
  if (p.dropout_p == 0.0f) return d;
  d.on = 1;
  d.k0 = static_cast<uint32_t>(p.dropout_seed & 0xffffffffu);
  d.k1 = static_cast<uint32_t>(p.dropout_seed >> 32);
  d.stream = 2u * p.dropout_layer + branch;
  d.t = static_cast<uint32_t>(floor(static_cast<double>(p.dropout_p) * 4294967296.0));
  d.scale = 1.0f / (1.0f - p.dropout_p);
  return d;
}

struct SavedLayout {
  size_t off[PTB_SAVED_COUNT];
  size_t total;
};

SavedLayout saved_layout(const Shape& s) {
  SavedLayout L;
  size_t o = 0;
  auto put = [&](int slot, size_t bytes) { L.off[slot] = o; o = align_up(o + bytes); };
  put(PTB_SAVED_A, s.T * s.h * 2);
  put(PTB_SAVED_MU, s.T * 4);
  put(PTB_SAVED_RSTD, s.T * 4);
  put(PTB_SAVED_QKV, s.T * 3 * s.hl * 2);
  put(PTB_SAVED_U, s.T * s.f1 * 2);
  put(PTB_SAVED_G, s.T * s.f * 2);
  put(PTB_SAVED_C, s.T * s.hl * 2);
  put(PTB_SAVED_LSE, s.b * s.n * s.s * 4);
  put(PTB_SAVED_A16, s.T * s.h * 2);
  put(PTB_SAVED_QK16, s.T * 2 * s.hl * 2);
  L.total = o;
  return L;
}

// Arrival counters one launch of the layer needs at most: output tiles of
// the largest GEMM launch, rows of the attention launches.
int max_gemm_tiles(const Shape& s) {
  const int T = static_cast<int>(s.T), h = static_cast<int>(s.h), hl = static_cast<int>(s.hl);
  const int K2 = static_cast<int>(s.K2), N1 = static_cast<int>(s.N1), f = static_cast<int>(s.f);
  int m = ptb::gemm_tiles(T, 2 * hl) + ptb::gemm_tiles(T, hl + static_cast<int>(s.f1));
  for (int t : {ptb::gemm_tiles(T, h), ptb::gemm_tiles(T, K2), ptb::gemm_tiles(K2, h),
                ptb::gemm_tiles(h, N1)})
    m = t > m ? t : m;
  // attention: one counter per (batch, head, row of 128)
  const long rows = s.b * s.n * ((s.s + 127) / 128);
  return rows > m ? static_cast<int>(rows) : m;
}

struct WorkLayout {
  size_t gemm_partials, counters, dc, dz, da, delta, partials, dym, wqk16, total;
  int max_tiles;
};

// Bytes of the fp16 copy of W_qkv's q and k columns, [h, 2 h_l].
size_t wqk16_bytes(const Shape& s) { return static_cast<size_t>(s.h) * 2 * s.hl * 2; }

// GEMM partial tiles and counters first (forward and backward), then the
// backward's intermediate gradients; the forward's fp16 copy of the q, k
// weight columns lies over the latter (the forward is done with it before
// the backward starts).
WorkLayout work_layout(const Shape& s) {
  WorkLayout W;
  size_t o = 0;
  W.max_tiles = max_gemm_tiles(s);
  W.gemm_partials = o; o = align_up(o + ptb::kGemmPartialBytes);
  W.counters = o; o = align_up(o + static_cast<size_t>(W.max_tiles) * 4);
  W.wqk16 = o;
  W.dc = o; o = align_up(o + s.T * s.hl * 2);
  W.dz = o; o = align_up(o + s.T * s.N1 * 2);
  W.da = o; o = align_up(o + s.T * s.h * 2);
  W.delta = o; o = align_up(o + s.b * s.n * s.s * 4);
  W.partials = o; o = align_up(o + static_cast<size_t>(ptb::layernorm_bwd_blocks(s.T)) * 2 * s.h * 4);
  W.dym = o; o = align_up(o + s.T * s.h * 2);  // dropout of dy (the branch output's gradient)
  W.total = std::max(o, align_up(W.wqk16 + wqk16_bytes(s)));
  return W;
}

// The serial block's stash (ptb_serial_saved_slot order).
struct SerialSavedLayout {
  size_t off[PTB_SERIAL_SAVED_COUNT];
  size_t total;
};

SerialSavedLayout serial_saved_layout(const Shape& s) {
  SerialSavedLayout L;
  size_t o = 0;
  auto put = [&](int slot, size_t bytes) { L.off[slot] = o; o = align_up(o + bytes); };
  put(PTB_SERIAL_A1, s.T * s.h * 2);
  put(PTB_SERIAL_MU1, s.T * 4);
  put(PTB_SERIAL_RSTD1, s.T * 4);
  put(PTB_SERIAL_A1_16, s.T * s.h * 2);
  put(PTB_SERIAL_QKV, s.T * 3 * s.hl * 2);
  put(PTB_SERIAL_QK16, s.T * 2 * s.hl * 2);
  put(PTB_SERIAL_C, s.T * s.hl * 2);
  put(PTB_SERIAL_LSE, s.b * s.n * s.s * 4);
  put(PTB_SERIAL_X1, s.T * s.h * 2);
  put(PTB_SERIAL_A2, s.T * s.h * 2);
  put(PTB_SERIAL_MU2, s.T * 4);
  put(PTB_SERIAL_RSTD2, s.T * 4);
  put(PTB_SERIAL_U, s.T * s.f1 * 2);
  put(PTB_SERIAL_G, s.T * s.f * 2);
  L.total = o;
  return L;
}

// Arrival counters one launch of the serial block needs at most.
int serial_max_tiles(const Shape& s) {
  const int T = static_cast<int>(s.T), h = static_cast<int>(s.h), hl = static_cast<int>(s.hl);
  const int f = static_cast<int>(s.f);
  int m = ptb::gemm_tiles(T, 2 * hl) + ptb::gemm_tiles(T, hl);
  const int f1 = static_cast<int>(s.f1);
  for (int t : {ptb::gemm_tiles(T, h), ptb::gemm_tiles(T, f1), ptb::gemm_tiles(f, h),
                ptb::gemm_tiles(h, f1), ptb::gemm_tiles(T, hl), ptb::gemm_tiles(hl, h),
                ptb::gemm_tiles(h, 3 * hl)})
    m = t > m ? t : m;
  const long rows = s.b * s.n * ((s.s + 127) / 128);
  return rows > m ? static_cast<int>(rows) : m;
}

// The serial block's scratch: GEMM partial tiles and counters first (all the
// forward needs), then the backward's intermediate gradients.  da holds the
// LN2 input gradient, then the LN1 one.
struct SerialWorkLayout {
  size_t gemm_partials, counters, du, da, dx1, dc, dz, delta, partials, dym, wqk16, total;
  int max_tiles;
};

SerialWorkLayout serial_work_layout(const Shape& s) {
  SerialWorkLayout W;
  size_t o = 0;
  W.max_tiles = serial_max_tiles(s);
  W.gemm_partials = o; o = align_up(o + ptb::kGemmPartialBytes);
  W.counters = o; o = align_up(o + static_cast<size_t>(W.max_tiles) * 4);
  W.wqk16 = o;  // forward only, over the backward's region
  W.du = o; o = align_up(o + s.T * s.f1 * 2);
  W.da = o; o = align_up(o + s.T * s.h * 2);
  W.dx1 = o; o = align_up(o + s.T * s.h * 2);
  W.dc = o; o = align_up(o + s.T * s.hl * 2);
  W.dz = o; o = align_up(o + s.T * 3 * s.hl * 2);
  W.delta = o; o = align_up(o + s.b * s.n * s.s * 4);
  W.partials = o; o = align_up(o + static_cast<size_t>(ptb::layernorm_bwd_blocks(s.T)) * 2 * s.h * 4);
  W.dym = o; o = align_up(o + s.T * s.h * 2);  // dropout of dy, then of dx1
  W.total = std::max(o, align_up(W.wqk16 + wqk16_bytes(s)));
  return W;
}

// ---- FP8 variant.  Every FP8 product reads two k-contiguous operands whose
// k extent is padded with zero codes to a multiple of 128 (one stage tile).
size_t pad128(size_t v) { return (v + 127) & ~static_cast<size_t>(127); }
size_t pad64(size_t v) { return (v + 63) & ~static_cast<size_t>(63); }

// One FP8 copy of an operand: `rows` rows of codes, contraction extent k
// padded to kp = pad128(k), and under block scaling its scale words
// (mx_scale_byte layout) [kp / 128][pad128(rows)] words.
struct Fp8Copy {
  size_t codes, scales;  // byte offsets (scales: SIZE_MAX when absent)
  size_t rows, kp;
};
// Appends a copy at offset *o.
Fp8Copy add_copy(size_t* o, size_t rows, size_t k, bool mx) {
  Fp8Copy c;
  c.rows = rows;
  c.kp = pad128(k);
  c.codes = *o;
  *o = align_up(*o + rows * c.kp);
  c.scales = SIZE_MAX;
  if (mx) {
    c.scales = *o;
    *o = align_up(*o + c.kp / 128 * pad128(rows) * sizeof(uint32_t));
  }
  return c;
}

// The FP8 weight buffer: amax of W1 = [W_qkv | W_fc1] and W2 = [W_o ; W_fc2]
// (current scaling), then both orientations of each in E4M3 (with their
// block scales under MX).
struct Fp8WeightLayout {
  size_t amax;
  Fp8Copy w1t, w1r, w2t, w2r;
  size_t total;
};
Fp8WeightLayout fp8_weight_layout(const Shape& s, bool mx) {
  Fp8WeightLayout L;
  size_t o = 0;
  L.amax = SIZE_MAX;
  if (!mx) { L.amax = o; o = align_up(o + 2 * sizeof(float)); }
  L.w1t = add_copy(&o, s.N1, s.h, mx);   // W1^T [N1, h]   (forward)
  L.w1r = add_copy(&o, s.h, s.N1, mx);   // W1   [h, N1]   (dgrad)
  L.w2t = add_copy(&o, s.h, s.K2, mx);   // W2^T [h, K2]   (forward)
  L.w2r = add_copy(&o, s.K2, s.h, mx);   // W2   [K2, h]   (dgrad)
  L.total = o;
  return L;
}

// The FP8 workspace: the bf16 layer's workspace, then the amax of the
// gradient operands (current scaling) and the FP8 copies that live within
// one call.
enum Fp8Amax { AMAX_DY = 0, AMAX_DZ, AMAX_COUNT };
struct Fp8WorkLayout {
  WorkLayout base;
  size_t amax;
  Fp8Copy a8, cg8, dy8, dy8t, dz8, dz8t;
  size_t total;
};
Fp8WorkLayout fp8_work_layout(const Shape& s, bool mx) {
  Fp8WorkLayout W;
  W.base = work_layout(s);
  size_t o = W.base.total;
  W.amax = o; o = align_up(o + AMAX_COUNT * sizeof(float));
  W.a8 = add_copy(&o, s.T, s.h, mx);     // a       [T, h]  (forward)
  W.cg8 = add_copy(&o, s.T, s.K2, mx);   // [c | g] [T, K2] (forward)
  W.dy8 = add_copy(&o, s.T, s.h, mx);    // dy      [T, h]
  W.dy8t = add_copy(&o, s.h, s.T, mx);   // dy^T    [h, T]
  W.dz8 = add_copy(&o, s.T, s.N1, mx);   // dZ      [T, N1]
  W.dz8t = add_copy(&o, s.N1, s.T, mx);  // dZ^T    [N1, T]
  W.total = o;
  return W;
}

// The FP8 layer's stash: the parallel block's slots, then what the forward
// casts for the weight gradients (the transposed E4M3 copies of a and
// [c | g] and their amax or block scales).
struct Fp8SavedLayout {
  SavedLayout base;
  size_t amax;
  Fp8Copy a8t, cg8t;
  size_t total;
};
Fp8SavedLayout fp8_saved_layout(const Shape& s, bool mx) {
  Fp8SavedLayout L;
  L.base = saved_layout(s);
  size_t o = L.base.total;
  L.amax = o; o = align_up(o + 2 * sizeof(float));   // amax of a, of [c | g]
  L.a8t = add_copy(&o, s.h, s.T, mx);                // a^T       [h, T]
  L.cg8t = add_copy(&o, s.K2, s.T, mx);              // [c | g]^T [K2, T]
  L.total = o;
  return L;
}

// The variant covers LayerNorm or RMSNorm with the GeLU MLP, under either
// recipe.
int32_t check_fp8_dims(const ptb_dims* dims, int32_t recipe, Shape* s) {
  const int32_t st = check_dims(dims, s);
  if (st != PTB_OK) return st;
  if (s->swiglu || dims->dropout_p != 0.0f || (recipe != PTB_FP8_CURRENT && recipe != PTB_FP8_MX))
    return PTB_ERR_ARG;
  // FP8 operands are addressed with 32-bit byte offsets as well: every copy
  // (rows x padded contiguous dimension, one byte each) stays below 2^31
  const size_t T = s->T, h = s->h, N1 = s->N1, K2 = s->K2;
  const size_t sizes[] = {T * pad128(h),  T * pad128(K2), T * pad128(N1), h * pad128(T),
                          K2 * pad128(T), N1 * pad128(T), N1 * pad128(h), h * pad128(N1),
                          h * pad128(K2), K2 * pad128(h)};
  for (size_t b : sizes)
    if (b >= (1UL << 31)) return PTB_ERR_DIMS;
  return PTB_OK;
}

constexpr int kOneSegment = 1 << 30;

ptb::CastSrc cast_one(const void* p, long ld, long R, long C) {
  const u16* q = static_cast<const u16*>(p);
  return ptb::CastSrc{q, q, static_cast<int>(ld), static_cast<int>(ld), kOneSegment, 0,
                      static_cast<int>(R), static_cast<int>(C)};
}
ptb::CastSrc cast_two(const void* p0, long ld0, const void* p1, long ld1, long split,
                      int on_rows, long R, long C) {
  return ptb::CastSrc{static_cast<const u16*>(p0), static_cast<const u16*>(p1),
                      static_cast<int>(ld0), static_cast<int>(ld1), static_cast<int>(split),
                      on_rows, static_cast<int>(R), static_cast<int>(C)};
}

// An FP8 operand [rows, ld] (bytes, k-contiguous).
ptb::Operand one8(const uint8_t* p, long ld, long rows) {
  const u16* q = reinterpret_cast<const u16*>(p);
  const uint32_t bytes = static_cast<uint32_t>(ld * rows);
  return ptb::Operand{q, q, static_cast<int>(ld), static_cast<int>(ld), INT_MAX, 0, bytes, bytes};
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr) return PTB_ERR_NULL;
  for (const void* p : ps)
    if (!aligned16(p)) return PTB_ERR_ALIGN;
  return PTB_OK;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }
template <typename T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

// A GEMM operand: row-major segments with leading dimension ld and `rows` rows.
ptb::Operand one(const u16* p, long ld, long rows) {
  const uint32_t bytes = static_cast<uint32_t>(ld * rows * 2);
  return ptb::Operand{p, p, static_cast<int>(ld), static_cast<int>(ld), INT_MAX, 0, bytes, bytes};
}
ptb::Operand two(const u16* p0, long ld0, long rows0, const u16* p1, long ld1, long rows1,
                 long split, int on_k) {
  return ptb::Operand{p0, p1, static_cast<int>(ld0), static_cast<int>(ld1),
                      static_cast<int>(split), on_k, static_cast<uint32_t>(ld0 * rows0 * 2),
                      static_cast<uint32_t>(ld1 * rows1 * 2)};
}
// Bytes spanned by `rows` rows of `width` elements at leading dimension ld
// (a column block of a wider matrix).
uint32_t view_bytes(long ld, long rows, long width) {
  return static_cast<uint32_t>(((rows - 1) * ld + width) * 2);
}

// amax of x into *amax (zero on entry), then its FP8 copies.
hipError_t cast_fp8(const ptb::CastSrc& x, ptb::Fp8Format fmt, float* amax, uint8_t* rows,
                    size_t ldr, uint8_t* cols, size_t ldc, hipStream_t strm) {
  const hipError_t e = ptb::launch_amax(x, amax, strm);
  if (e != hipSuccess) return e;
  return ptb::launch_cast_fp8(x, fmt, amax, rows, static_cast<int>(ldr), cols,
                              static_cast<int>(ldc), strm);
}

#define PTB_HIP(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return PTB_ERR_HIP;  \
  } while (0)

// An FP8 copy in a caller buffer: codes [rows][kp] and, under block
// scaling, scale words [kp / 128][pad128(rows)] (mx_scale_byte layout).
struct Copy8 {
  uint8_t* q;
  uint32_t* s;
  size_t ld;   // kp
  int sld;     // pad128(rows)
  size_t rows;
};
Copy8 copy_at(void* base, const Fp8Copy& c) {
  return Copy8{at<uint8_t>(base, c.codes),
               c.scales == SIZE_MAX ? nullptr : at<uint32_t>(base, c.scales), c.kp,
               static_cast<int>(pad128(c.rows)), c.rows};
}
Copy8 copy_at(const void* base, const Fp8Copy& c) {
  return copy_at(const_cast<void*>(base), c);
}

// The two FP8 copies of x under the layer's recipe (rows: contraction along
// x's columns; cols: the transpose).  Current scaling: amax of x into
// *amax (zero on entry), then the cast; block scaling: one pass.
hipError_t cast_copies(bool mx, const ptb::CastSrc& x, ptb::Fp8Format fmt, float* amax,
                       const Copy8& rows, const Copy8& cols, hipStream_t strm) {
  if (mx)
    return ptb::launch_cast_mx(x, fmt, rows.q, static_cast<int>(rows.ld), rows.s, rows.sld,
                               cols.q, static_cast<int>(cols.ld), cols.s, cols.sld, strm);
  return cast_fp8(x, fmt, amax, rows.q, rows.ld, cols.q, cols.ld, strm);
}

// An FP8 product C = A B^T of two copies (A [M][K], B [N][K]) with the
// problem's epilogue, scaled by the operands' amax or block scales.
hipError_t gemm8(bool mx, ptb::GemmProblem pr, const Copy8& a, ptb::Fp8Format fa,
                 const float* amax_a, const Copy8& b, ptb::Fp8Format fb, const float* amax_b,
                 ptb::EpiMode mode, const ptb::GemmScratch& gs, hipStream_t strm) {
  pr.M = static_cast<int>(a.rows);
  pr.N = static_cast<int>(b.rows);
  pr.K = static_cast<int>(a.ld);
  pr.A = one8(a.q, a.ld, a.rows);
  pr.B = one8(b.q, b.ld, b.rows);
  if (mx)
    return ptb::launch_gemm_mx(pr, fa, ptb::MxScales{a.s, a.sld}, fb, ptb::MxScales{b.s, b.sld},
                               mode, gs, strm);
  return ptb::launch_gemm_fp8(pr, fa, amax_a, fb, amax_b, mode, gs, strm);
}


// Enqueue one stage, bracketed by the caller's timing events when given.
#define PTB_STAGE(i, expr)                                                          \
  do {                                                                              \
    if (ev != nullptr && ev[2 * (i)] != nullptr)                                    \
      PTB_HIP(hipEventRecord(static_cast<hipEvent_t>(ev[2 * (i)]), strm));           \
    PTB_HIP(expr);                                                                  \
    if (ev != nullptr && ev[2 * (i) + 1] != nullptr)                                \
      PTB_HIP(hipEventRecord(static_cast<hipEvent_t>(ev[2 * (i) + 1]), strm));       \
  } while (0)

}  // namespace

extern "C" {

int32_t ptb_abi_version(void) { return PTB_ABI_VERSION; }

const char* ptb_status_string(int32_t status) {
  switch (status) {
    case PTB_OK: return "ok";
    case PTB_ERR_NULL: return "a required pointer is NULL";
    case PTB_ERR_DIMS: return "invalid or too large dimensions";
    case PTB_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case PTB_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PTB_ERR_WINDOW: return "window must be >= 1";
    case PTB_ERR_EPS: return "ln_eps must be a finite positive number";
    case PTB_ERR_HIP: return "a HIP kernel launch failed";
    case PTB_ERR_ARG: return "invalid layer variant, optimizer hyper-parameters or tensor list";
    case PTB_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int32_t ptb_validate_dims(const ptb_dims* dims) { return check_dims(dims, nullptr); }

int32_t ptb_saved_bytes(const ptb_dims* dims, size_t* bytes) {
  Shape s;
  const int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = saved_layout(s).total;
  return PTB_OK;
}

int32_t ptb_workspace_bytes(const ptb_dims* dims, size_t* bytes) {
  Shape s;
  const int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = work_layout(s).total;
  return PTB_OK;
}

int32_t ptb_saved_layout(const ptb_dims* dims, size_t* offsets) {
  Shape s;
  const int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  if (offsets == nullptr) return PTB_ERR_NULL;
  const SavedLayout L = saved_layout(s);
  for (int i = 0; i < PTB_SAVED_COUNT; ++i) offsets[i] = L.off[i];
  return PTB_OK;
}

int32_t ptb_forward_timed(const ptb_dims* dims, const void* x, const void* ln_gamma,
                          const void* ln_beta, const void* w_qkv, const void* w_o,
                          const void* w_fc1, const void* w_fc2, void* y, void* saved,
                          void* workspace, void* stream, void* const* ev) {
  Shape s;
  int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({x, ln_gamma, ln_beta, w_qkv, w_o, w_fc1, w_fc2, y, saved, workspace});
  if (st != PTB_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const SavedLayout L = saved_layout(s);
  const WorkLayout W = work_layout(s);
  const ptb::GemmScratch gs{at<float>(workspace, W.gemm_partials),
                            at<int>(workspace, W.counters), W.max_tiles};
  u16* a = at<u16>(saved, L.off[PTB_SAVED_A]);
  float* mu = at<float>(saved, L.off[PTB_SAVED_MU]);
  float* rstd = at<float>(saved, L.off[PTB_SAVED_RSTD]);
  u16* qkv = at<u16>(saved, L.off[PTB_SAVED_QKV]);
  u16* u = at<u16>(saved, L.off[PTB_SAVED_U]);
  u16* g = at<u16>(saved, L.off[PTB_SAVED_G]);
  u16* c = at<u16>(saved, L.off[PTB_SAVED_C]);
  float* lse = at<float>(saved, L.off[PTB_SAVED_LSE]);
  u16* a16 = at<u16>(saved, L.off[PTB_SAVED_A16]);
  u16* qk16 = at<u16>(saved, L.off[PTB_SAVED_QK16]);
  u16* wqk16 = at<u16>(workspace, W.wqk16);
  const u16* X = static_cast<const u16*>(x);
  const u16* Wqkv = static_cast<const u16*>(w_qkv);

  // the LayerNorm launch also clears the arrival counters of the launches after it
  PTB_STAGE(0, ptb::launch_layernorm_fwd(X, static_cast<const u16*>(ln_gamma),
                                    static_cast<const u16*>(ln_beta), a, a16, mu, rstd,
                                    static_cast<int>(s.T), static_cast<int>(s.h), dims->ln_eps,
                                    strm, s.rms, gs.counters, gs.max_tiles));
  PTB_STAGE(1, ptb::launch_cast_f16(Wqkv, static_cast<int>(3 * s.hl), static_cast<int>(s.h),
                                    static_cast<int>(2 * s.hl), wqk16,
                                    static_cast<int>(2 * s.hl), strm));
  {  // [QKV | FC1] projection in one launch of two products:
     //   [q | k] = a16 x W_q|k in fp16 (stored in bf16 and in fp16)
     //   [v | u] = a x [W_v | W_fc1], with g = GeLU(u) on the FC1 columns
     //   (SwiGLU: u = [u1 | u3] in 32-column blocks, g = silu(u1) * u3)
    ptb::Epilogue e{};
    e.o0 = qkv; e.ld0 = static_cast<int>(3 * s.hl);
    e.o1 = u; e.o2 = g; e.ld1 = static_cast<int>(s.f1); e.ld2 = static_cast<int>(s.f);
    e.o3 = qk16; e.ld3 = static_cast<int>(2 * s.hl); e.lo_cols = static_cast<int>(2 * s.hl);
    e.split = static_cast<int>(3 * s.hl);
    ptb::GemmProblem pr[2];
    pr[0].M = static_cast<int>(s.T); pr[0].N = static_cast<int>(2 * s.hl);
    pr[0].K = static_cast<int>(s.h);
    pr[0].A = one(a16, s.h, s.T);
    pr[0].B = one(wqk16, 2 * s.hl, s.h);
    pr[0].epi = e;
    pr[0].epi.col_base = 0;
    pr[1].M = static_cast<int>(s.T); pr[1].N = static_cast<int>(s.hl + s.f1);
    pr[1].K = static_cast<int>(s.h);
    pr[1].A = one(a, s.h, s.T);
    pr[1].B = two(Wqkv + 2 * s.hl, 3 * s.hl, s.h, static_cast<const u16*>(w_fc1), s.f1, s.h,
                  s.hl, 0);
    pr[1].B.bytes0 = view_bytes(3 * s.hl, s.h, s.hl);
    pr[1].epi = e;
    pr[1].epi.col_base = static_cast<int>(2 * s.hl);
    PTB_STAGE(2, ptb::launch_gemm_group(pr, 2, ptb::KMAJOR, ptb::OUTER_MAJOR,
                                        s.swiglu ? ptb::EPI_QKV_SWIGLU : ptb::EPI_QKV_GELU, gs,
                                        strm, /*f16_prob0=*/true));
  }
  const ptb::AttnScratch as{gs.partials, ptb::kGemmPartialBytes / sizeof(float), gs.counters,
                            gs.max_tiles, ptb::device_compute_units()};
  PTB_STAGE(3, ptb::launch_attention_fwd(qkv, qk16, c, lse, static_cast<int>(s.b),
                                    static_cast<int>(s.s), static_cast<int>(s.n),
                                    static_cast<int>(s.d), static_cast<int>(s.w), as, strm));
  {  // [O ; FC2] projection plus the residual
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(y); e.i0 = X; e.ld0 = static_cast<int>(s.h);
    e.drop = dropout_of(*dims, 0);  // y = x + D * (Attn + MLP)
    PTB_STAGE(4, ptb::launch_gemm(
        static_cast<int>(s.T), static_cast<int>(s.h), static_cast<int>(s.K2),
        two(c, s.hl, s.T, g, s.f, s.T, s.hl, 1), ptb::KMAJOR,
        two(static_cast<const u16*>(w_o), s.h, s.hl, static_cast<const u16*>(w_fc2), s.h, s.f,
            s.hl, 1),
        ptb::OUTER_MAJOR, ptb::EPI_RESIDUAL, e, gs, strm));
  }
  return PTB_OK;
}

int32_t ptb_backward_timed(const ptb_dims* dims, const void* dy, const void* x,
                           const void* ln_gamma, const void* w_qkv, const void* w_o,
                           const void* w_fc1, const void* w_fc2, const void* saved, void* dx,
                           void* d_ln_gamma, void* d_ln_beta, void* dw_qkv, void* dw_o,
                           void* dw_fc1, void* dw_fc2, void* workspace, void* stream,
                           void* const* ev) {
  Shape s;
  int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({dy, x, ln_gamma, w_qkv, w_o, w_fc1, w_fc2, saved, dx, d_ln_gamma, d_ln_beta,
                   dw_qkv, dw_o, dw_fc1, dw_fc2, workspace});
  if (st != PTB_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const SavedLayout L = saved_layout(s);
  const WorkLayout W = work_layout(s);
  const u16* a = at<u16>(saved, L.off[PTB_SAVED_A]);
  const float* mu = at<float>(saved, L.off[PTB_SAVED_MU]);
  const float* rstd = at<float>(saved, L.off[PTB_SAVED_RSTD]);
  const u16* qkv = at<u16>(saved, L.off[PTB_SAVED_QKV]);
  const u16* u = at<u16>(saved, L.off[PTB_SAVED_U]);
  const u16* g = at<u16>(saved, L.off[PTB_SAVED_G]);
  const u16* c = at<u16>(saved, L.off[PTB_SAVED_C]);
  const float* lse = at<float>(saved, L.off[PTB_SAVED_LSE]);
  const u16* qk16 = at<u16>(saved, L.off[PTB_SAVED_QK16]);
  u16* dc = at<u16>(workspace, W.dc);
  u16* dz = at<u16>(workspace, W.dz);
  u16* da = at<u16>(workspace, W.da);
  float* delta = at<float>(workspace, W.delta);
  float* partials = at<float>(workspace, W.partials);
  const ptb::GemmScratch gs{at<float>(workspace, W.gemm_partials),
                            at<int>(workspace, W.counters), W.max_tiles};
  const u16* DY = static_cast<const u16*>(dy);
  const int T = static_cast<int>(s.T), h = static_cast<int>(s.h);
  // the gradient of the branch output: dy, or D * dy under dropout (the
  // mask regenerated from its key); the residual path takes dy itself
  const ptb::Dropout drop = dropout_of(*dims, 0);
  u16* dym = at<u16>(workspace, W.dym);
  const u16* DB = drop.on ? dym : DY;

  PTB_HIP(ptb::launch_zero_i32(gs.counters, gs.max_tiles, strm));

  {  // dgrad through [O ; FC2]: dc, and du = dg * GeLU'(u) into dZ's FC1 columns
     // (SwiGLU: du1 = dg * u3 * silu'(u1), du3 = dg * silu(u1))
    ptb::Epilogue e{};
    e.o0 = dc; e.ld0 = static_cast<int>(s.hl);
    e.o1 = dz; e.ld1 = static_cast<int>(s.N1); e.col_off1 = static_cast<int>(3 * s.hl);
    e.i0 = u; e.ld2 = static_cast<int>(s.f1);
    e.split = static_cast<int>(s.hl);
    auto stage0 = [&]() -> hipError_t {
      if (drop.on) {
        const hipError_t er = ptb::launch_dropout_apply(DY, dym, s.T * s.h, drop, strm);
        if (er != hipSuccess) return er;
      }
      return ptb::launch_gemm(
          T, static_cast<int>(s.K2), h, one(DB, s.h, s.T), ptb::KMAJOR,
          two(static_cast<const u16*>(w_o), s.h, s.hl, static_cast<const u16*>(w_fc2), s.h, s.f,
              s.hl, 0),
          ptb::KMAJOR, s.swiglu ? ptb::EPI_DSWIGLU : ptb::EPI_DGELU, e, gs, strm);
    };
    PTB_STAGE(0, stage0());
  }
  const ptb::AttnScratch as{gs.partials, ptb::kGemmPartialBytes / sizeof(float), gs.counters,
                            gs.max_tiles, ptb::device_compute_units()};
  PTB_STAGE(1, ptb::launch_attention_bwd(qkv, qk16, c, lse, dc, delta, dz, static_cast<int>(s.N1),
                                    static_cast<int>(s.b), static_cast<int>(s.s),
                                    static_cast<int>(s.n), static_cast<int>(s.d),
                                    static_cast<int>(s.w), as, strm));
  {  // wgrad of [O ; FC2]: [c | g]^T dy
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(dw_o); e.ld0 = h;
    e.o1 = static_cast<u16*>(dw_fc2); e.ld1 = h;
    e.split = static_cast<int>(s.hl);
    PTB_STAGE(2, ptb::launch_gemm(static_cast<int>(s.K2), h, T, two(c, s.hl, s.T, g, s.f, s.T, s.hl, 0),
                             ptb::OUTER_MAJOR, one(DB, s.h, s.T), ptb::OUTER_MAJOR,
                             ptb::EPI_STORE2_ROWS, e, gs, strm));
  }
  {  // dgrad through [QKV | FC1]: da = dZ [W_qkv | W_fc1]^T
    ptb::Epilogue e{};
    e.o0 = da; e.ld0 = h;
    e.split = h;  // one output
    PTB_STAGE(3, ptb::launch_gemm(
        T, h, static_cast<int>(s.N1), one(dz, s.N1, s.T), ptb::KMAJOR,
        two(static_cast<const u16*>(w_qkv), 3 * s.hl, s.h, static_cast<const u16*>(w_fc1), s.f1,
            s.h, 3 * s.hl, 1),
        ptb::KMAJOR, ptb::EPI_STORE2_COLS, e, gs, strm));
  }
  {  // wgrad of [QKV | FC1]: a^T dZ
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(dw_qkv); e.ld0 = static_cast<int>(3 * s.hl);
    e.o1 = static_cast<u16*>(dw_fc1); e.ld1 = static_cast<int>(s.f1);
    e.split = static_cast<int>(3 * s.hl);
    PTB_STAGE(4, ptb::launch_gemm(h, static_cast<int>(s.N1), T, one(a, s.h, s.T), ptb::OUTER_MAJOR,
                             one(dz, s.N1, s.T), ptb::OUTER_MAJOR, ptb::EPI_STORE2_COLS, e, gs,
                             strm));
  }
  PTB_STAGE(5, ptb::launch_layernorm_bwd(da, static_cast<const u16*>(x),
                                    static_cast<const u16*>(ln_gamma), mu, rstd, DY,
                                    static_cast<u16*>(dx), partials,
                                    static_cast<u16*>(d_ln_gamma), static_cast<u16*>(d_ln_beta),
                                    T, h, strm, s.rms));
  return PTB_OK;
}

int32_t ptb_forward(const ptb_dims* dims, const void* x, const void* ln_gamma,
                    const void* ln_beta, const void* w_qkv, const void* w_o, const void* w_fc1,
                    const void* w_fc2, void* y, void* saved, void* workspace, void* stream) {
  return ptb_forward_timed(dims, x, ln_gamma, ln_beta, w_qkv, w_o, w_fc1, w_fc2, y, saved,
                           workspace, stream, nullptr);
}

int32_t ptb_backward(const ptb_dims* dims, const void* dy, const void* x, const void* ln_gamma,
                     const void* w_qkv, const void* w_o, const void* w_fc1, const void* w_fc2,
                     const void* saved, void* dx, void* d_ln_gamma, void* d_ln_beta,
                     void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2, void* workspace,
                     void* stream) {
  return ptb_backward_timed(dims, dy, x, ln_gamma, w_qkv, w_o, w_fc1, w_fc2, saved, dx,
                            d_ln_gamma, d_ln_beta, dw_qkv, dw_o, dw_fc1, dw_fc2, workspace,
                            stream, nullptr);
}

int32_t ptb_serial_saved_bytes(const ptb_dims* dims, size_t* bytes) {
  Shape s;
  const int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = serial_saved_layout(s).total;
  return PTB_OK;
}

int32_t ptb_serial_workspace_bytes(const ptb_dims* dims, size_t* bytes) {
  Shape s;
  const int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = serial_work_layout(s).total;
  return PTB_OK;
}

int32_t ptb_serial_saved_layout(const ptb_dims* dims, size_t* offsets) {
  Shape s;
  const int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  if (offsets == nullptr) return PTB_ERR_NULL;
  const SerialSavedLayout L = serial_saved_layout(s);
  for (int i = 0; i < PTB_SERIAL_SAVED_COUNT; ++i) offsets[i] = L.off[i];
  return PTB_OK;
}

int32_t ptb_serial_forward_timed(const ptb_dims* dims, const void* x, const void* ln1_gamma,
                                 const void* ln1_beta, const void* ln2_gamma,
                                 const void* ln2_beta, const void* w_qkv, const void* w_o,
                                 const void* w_fc1, const void* w_fc2, void* y, void* saved,
                                 void* workspace, void* stream, void* const* ev) {
  Shape s;
  int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({x, ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, w_qkv, w_o, w_fc1, w_fc2, y,
                   saved, workspace});
  if (st != PTB_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const SerialSavedLayout L = serial_saved_layout(s);
  const SerialWorkLayout W = serial_work_layout(s);
  const ptb::GemmScratch gs{at<float>(workspace, W.gemm_partials),
                            at<int>(workspace, W.counters), W.max_tiles};
  u16* a1 = at<u16>(saved, L.off[PTB_SERIAL_A1]);
  float* mu1 = at<float>(saved, L.off[PTB_SERIAL_MU1]);
  float* rstd1 = at<float>(saved, L.off[PTB_SERIAL_RSTD1]);
  u16* a1_16 = at<u16>(saved, L.off[PTB_SERIAL_A1_16]);
  u16* qkv = at<u16>(saved, L.off[PTB_SERIAL_QKV]);
  u16* qk16 = at<u16>(saved, L.off[PTB_SERIAL_QK16]);
  u16* wqk16 = at<u16>(workspace, W.wqk16);
  u16* c = at<u16>(saved, L.off[PTB_SERIAL_C]);
  float* lse = at<float>(saved, L.off[PTB_SERIAL_LSE]);
  u16* x1 = at<u16>(saved, L.off[PTB_SERIAL_X1]);
  u16* a2 = at<u16>(saved, L.off[PTB_SERIAL_A2]);
  float* mu2 = at<float>(saved, L.off[PTB_SERIAL_MU2]);
  float* rstd2 = at<float>(saved, L.off[PTB_SERIAL_RSTD2]);
  u16* u = at<u16>(saved, L.off[PTB_SERIAL_U]);
  u16* g = at<u16>(saved, L.off[PTB_SERIAL_G]);
  const u16* X = static_cast<const u16*>(x);
  const u16* Wqkv = static_cast<const u16*>(w_qkv);
  const int T = static_cast<int>(s.T), h = static_cast<int>(s.h);

  // the LayerNorm launch also clears the arrival counters of the launches after it
  PTB_STAGE(0, ptb::launch_layernorm_fwd(X, static_cast<const u16*>(ln1_gamma),
                                         static_cast<const u16*>(ln1_beta), a1, a1_16, mu1,
                                         rstd1, T, h, dims->ln_eps, strm, s.rms, gs.counters,
                                         gs.max_tiles));
  PTB_STAGE(1, ptb::launch_cast_f16(Wqkv, static_cast<int>(3 * s.hl), h,
                                    static_cast<int>(2 * s.hl), wqk16,
                                    static_cast<int>(2 * s.hl), strm));
  {  // QKV projection, one launch of two products: [q | k] = a1_16 x W_q|k in
     // fp16 (as in the parallel block) and v from a1
    ptb::Epilogue e{};
    e.o0 = qkv; e.ld0 = static_cast<int>(3 * s.hl);
    e.o3 = qk16; e.ld3 = static_cast<int>(2 * s.hl); e.lo_cols = static_cast<int>(2 * s.hl);
    e.split = static_cast<int>(3 * s.hl);
    ptb::GemmProblem pr[2];
    pr[0].M = T; pr[0].N = static_cast<int>(2 * s.hl); pr[0].K = h;
    pr[0].A = one(a1_16, s.h, s.T);
    pr[0].B = one(wqk16, 2 * s.hl, s.h);
    pr[0].epi = e;
    pr[0].epi.col_base = 0;
    pr[1].M = T; pr[1].N = static_cast<int>(s.hl); pr[1].K = h;
    pr[1].A = one(a1, s.h, s.T);
    pr[1].B = one(Wqkv + 2 * s.hl, 3 * s.hl, s.h);
    pr[1].B.bytes0 = pr[1].B.bytes1 = view_bytes(3 * s.hl, s.h, s.hl);
    pr[1].epi = e;
    pr[1].epi.col_base = static_cast<int>(2 * s.hl);
    PTB_STAGE(2, ptb::launch_gemm_group(pr, 2, ptb::KMAJOR, ptb::OUTER_MAJOR,
                                        ptb::EPI_QKV_GELU, gs, strm, /*f16_prob0=*/true));
  }
  const ptb::AttnScratch as{gs.partials, ptb::kGemmPartialBytes / sizeof(float), gs.counters,
                            gs.max_tiles, ptb::device_compute_units()};
  PTB_STAGE(3, ptb::launch_attention_fwd(qkv, qk16, c, lse, static_cast<int>(s.b),
                                         static_cast<int>(s.s), static_cast<int>(s.n),
                                         static_cast<int>(s.d), static_cast<int>(s.w), as, strm));
  {  // x1 = x + c W_o
    ptb::Epilogue e{};
    e.o0 = x1; e.i0 = X; e.ld0 = h;
    e.drop = dropout_of(*dims, 0);  // x1 = x + D1 * Attn W_o
    PTB_STAGE(4, ptb::launch_gemm(T, h, static_cast<int>(s.hl), one(c, s.hl, s.T), ptb::KMAJOR,
                                  one(static_cast<const u16*>(w_o), s.h, s.hl), ptb::OUTER_MAJOR,
                                  ptb::EPI_RESIDUAL, e, gs, strm));
  }
  PTB_STAGE(5, ptb::launch_layernorm_fwd(x1, static_cast<const u16*>(ln2_gamma),
                                         static_cast<const u16*>(ln2_beta), a2, nullptr, mu2,
                                         rstd2, T, h, dims->ln_eps, strm, s.rms));
  {  // u = a2 W_fc1, g = GeLU(u) (SwiGLU: silu(u1) * u3): every column on the
     // FC1 side of the split
    ptb::Epilogue e{};
    e.o1 = u; e.o2 = g; e.ld1 = static_cast<int>(s.f1); e.ld2 = static_cast<int>(s.f);
    e.split = 0; e.lo_cols = 0; e.col_base = 0;
    PTB_STAGE(6, ptb::launch_gemm(T, static_cast<int>(s.f1), h, one(a2, s.h, s.T), ptb::KMAJOR,
                                  one(static_cast<const u16*>(w_fc1), s.f1, s.h),
                                  ptb::OUTER_MAJOR,
                                  s.swiglu ? ptb::EPI_QKV_SWIGLU : ptb::EPI_QKV_GELU, e, gs,
                                  strm));
  }
  {  // y = x1 + g W_fc2
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(y); e.i0 = x1; e.ld0 = h;
    e.drop = dropout_of(*dims, 1);  // y = x1 + D2 * MLP
    PTB_STAGE(7, ptb::launch_gemm(T, h, static_cast<int>(s.f), one(g, s.f, s.T), ptb::KMAJOR,
                                  one(static_cast<const u16*>(w_fc2), s.h, s.f),
                                  ptb::OUTER_MAJOR, ptb::EPI_RESIDUAL, e, gs, strm));
  }
  return PTB_OK;
}

int32_t ptb_serial_backward_timed(const ptb_dims* dims, const void* dy, const void* x,
                                  const void* ln1_gamma, const void* ln2_gamma,
                                  const void* w_qkv, const void* w_o, const void* w_fc1,
                                  const void* w_fc2, const void* saved, void* dx,
                                  void* d_ln1_gamma, void* d_ln1_beta, void* d_ln2_gamma,
                                  void* d_ln2_beta, void* dw_qkv, void* dw_o, void* dw_fc1,
                                  void* dw_fc2, void* workspace, void* stream,
                                  void* const* ev) {
  Shape s;
  int32_t st = check_dims(dims, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({dy, x, ln1_gamma, ln2_gamma, w_qkv, w_o, w_fc1, w_fc2, saved, dx,
                   d_ln1_gamma, d_ln1_beta, d_ln2_gamma, d_ln2_beta, dw_qkv, dw_o, dw_fc1,
                   dw_fc2, workspace});
  if (st != PTB_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const SerialSavedLayout L = serial_saved_layout(s);
  const SerialWorkLayout W = serial_work_layout(s);
  const u16* a1 = at<u16>(saved, L.off[PTB_SERIAL_A1]);
  const float* mu1 = at<float>(saved, L.off[PTB_SERIAL_MU1]);
  const float* rstd1 = at<float>(saved, L.off[PTB_SERIAL_RSTD1]);
  const u16* qkv = at<u16>(saved, L.off[PTB_SERIAL_QKV]);
  const u16* qk16 = at<u16>(saved, L.off[PTB_SERIAL_QK16]);
  const u16* c = at<u16>(saved, L.off[PTB_SERIAL_C]);
  const float* lse = at<float>(saved, L.off[PTB_SERIAL_LSE]);
  const u16* x1 = at<u16>(saved, L.off[PTB_SERIAL_X1]);
  const u16* a2 = at<u16>(saved, L.off[PTB_SERIAL_A2]);
  const float* mu2 = at<float>(saved, L.off[PTB_SERIAL_MU2]);
  const float* rstd2 = at<float>(saved, L.off[PTB_SERIAL_RSTD2]);
  const u16* u = at<u16>(saved, L.off[PTB_SERIAL_U]);
  const u16* g = at<u16>(saved, L.off[PTB_SERIAL_G]);
  u16* du = at<u16>(workspace, W.du);
  u16* da = at<u16>(workspace, W.da);
  u16* dx1 = at<u16>(workspace, W.dx1);
  u16* dc = at<u16>(workspace, W.dc);
  u16* dz = at<u16>(workspace, W.dz);
  float* delta = at<float>(workspace, W.delta);
  float* partials = at<float>(workspace, W.partials);
  const ptb::GemmScratch gs{at<float>(workspace, W.gemm_partials),
                            at<int>(workspace, W.counters), W.max_tiles};
  const u16* DY = static_cast<const u16*>(dy);
  const int T = static_cast<int>(s.T), h = static_cast<int>(s.h);
  const int hl = static_cast<int>(s.hl), f = static_cast<int>(s.f);
  const int f1 = static_cast<int>(s.f1);
  // gradients of the two branch outputs under dropout: D2 * dy for the MLP,
  // D1 * dx1 for attention (masks regenerated from their keys, into dym one
  // after the other); the residual paths take dy and dx1 themselves
  const ptb::Dropout drop1 = dropout_of(*dims, 0), drop2 = dropout_of(*dims, 1);
  u16* dym = at<u16>(workspace, W.dym);
  const u16* DB2 = drop2.on ? dym : DY;
  const u16* DB1 = drop1.on ? dym : dx1;

  PTB_HIP(ptb::launch_zero_i32(gs.counters, gs.max_tiles, strm));
  {  // du = (D2 dy W_fc2^T) * GeLU'(u) (SwiGLU: du1, du3): every column on the
     // activation side of the split
    ptb::Epilogue e{};
    e.o1 = du; e.ld1 = f1; e.col_off1 = 0;
    e.i0 = u; e.ld2 = f1;
    e.split = 0;
    auto stage0 = [&]() -> hipError_t {
      if (drop2.on) {
        const hipError_t er = ptb::launch_dropout_apply(DY, dym, s.T * s.h, drop2, strm);
        if (er != hipSuccess) return er;
      }
      return ptb::launch_gemm(T, f, h, one(DB2, s.h, s.T), ptb::KMAJOR,
                              one(static_cast<const u16*>(w_fc2), s.h, s.f), ptb::KMAJOR,
                              s.swiglu ? ptb::EPI_DSWIGLU : ptb::EPI_DGELU, e, gs, strm);
    };
    PTB_STAGE(0, stage0());
  }
  {  // dW_fc2 = g^T (D2 dy)
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(dw_fc2); e.ld0 = h;
    e.split = f;  // one output
    PTB_STAGE(1, ptb::launch_gemm(f, h, T, one(g, s.f, s.T), ptb::OUTER_MAJOR, one(DB2, s.h, s.T),
                                  ptb::OUTER_MAJOR, ptb::EPI_STORE2_ROWS, e, gs, strm));
  }
  {  // da2 = du W_fc1^T
    ptb::Epilogue e{};
    e.o0 = da; e.ld0 = h;
    e.split = h;
    PTB_STAGE(2, ptb::launch_gemm(T, h, f1, one(du, s.f1, s.T), ptb::KMAJOR,
                                  one(static_cast<const u16*>(w_fc1), s.f1, s.h), ptb::KMAJOR,
                                  ptb::EPI_STORE2_COLS, e, gs, strm));
  }
  {  // dW_fc1 = a2^T du
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(dw_fc1); e.ld0 = f1;
    e.split = f1;
    PTB_STAGE(3, ptb::launch_gemm(h, f1, T, one(a2, s.h, s.T), ptb::OUTER_MAJOR,
                                  one(du, s.f1, s.T), ptb::OUTER_MAJOR, ptb::EPI_STORE2_COLS, e,
                                  gs, strm));
  }
  // dx1 = dy + LN2'(da2)
  PTB_STAGE(4, ptb::launch_layernorm_bwd(da, x1, static_cast<const u16*>(ln2_gamma), mu2, rstd2,
                                         DY, dx1, partials, static_cast<u16*>(d_ln2_gamma),
                                         static_cast<u16*>(d_ln2_beta), T, h, strm, s.rms));
  {  // dc = (D1 dx1) W_o^T
    ptb::Epilogue e{};
    e.o0 = dc; e.ld0 = hl;
    e.split = hl;
    auto stage5 = [&]() -> hipError_t {
      if (drop1.on) {
        const hipError_t er = ptb::launch_dropout_apply(dx1, dym, s.T * s.h, drop1, strm);
        if (er != hipSuccess) return er;
      }
      return ptb::launch_gemm(T, hl, h, one(DB1, s.h, s.T), ptb::KMAJOR,
                              one(static_cast<const u16*>(w_o), s.h, s.hl), ptb::KMAJOR,
                              ptb::EPI_STORE2_COLS, e, gs, strm);
    };
    PTB_STAGE(5, stage5());
  }
  {  // dW_o = c^T (D1 dx1)
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(dw_o); e.ld0 = h;
    e.split = hl;
    PTB_STAGE(6, ptb::launch_gemm(hl, h, T, one(c, s.hl, s.T), ptb::OUTER_MAJOR,
                                  one(DB1, s.h, s.T), ptb::OUTER_MAJOR, ptb::EPI_STORE2_ROWS, e,
                                  gs, strm));
  }
  const ptb::AttnScratch as{gs.partials, ptb::kGemmPartialBytes / sizeof(float), gs.counters,
                            gs.max_tiles, ptb::device_compute_units()};
  PTB_STAGE(7, ptb::launch_attention_bwd(qkv, qk16, c, lse, dc, delta, dz, 3 * hl,
                                         static_cast<int>(s.b), static_cast<int>(s.s),
                                         static_cast<int>(s.n), static_cast<int>(s.d),
                                         static_cast<int>(s.w), as, strm));
  {  // da1 = dZ W_qkv^T
    ptb::Epilogue e{};
    e.o0 = da; e.ld0 = h;
    e.split = h;
    PTB_STAGE(8, ptb::launch_gemm(T, h, 3 * hl, one(dz, 3 * s.hl, s.T), ptb::KMAJOR,
                                  one(static_cast<const u16*>(w_qkv), 3 * s.hl, s.h), ptb::KMAJOR,
                                  ptb::EPI_STORE2_COLS, e, gs, strm));
  }
  {  // dW_qkv = a1^T dZ
    ptb::Epilogue e{};
    e.o0 = static_cast<u16*>(dw_qkv); e.ld0 = 3 * hl;
    e.split = 3 * hl;
    PTB_STAGE(9, ptb::launch_gemm(h, 3 * hl, T, one(a1, s.h, s.T), ptb::OUTER_MAJOR,
                                  one(dz, 3 * s.hl, s.T), ptb::OUTER_MAJOR, ptb::EPI_STORE2_COLS,
                                  e, gs, strm));
  }
  // dx = dx1 + LN1'(da1)
  PTB_STAGE(10, ptb::launch_layernorm_bwd(da, static_cast<const u16*>(x),
                                          static_cast<const u16*>(ln1_gamma), mu1, rstd1, dx1,
                                          static_cast<u16*>(dx), partials,
                                          static_cast<u16*>(d_ln1_gamma),
                                          static_cast<u16*>(d_ln1_beta), T, h, strm, s.rms));
  return PTB_OK;
}

int32_t ptb_serial_forward(const ptb_dims* dims, const void* x, const void* ln1_gamma,
                           const void* ln1_beta, const void* ln2_gamma, const void* ln2_beta,
                           const void* w_qkv, const void* w_o, const void* w_fc1,
                           const void* w_fc2, void* y, void* saved, void* workspace,
                           void* stream) {
  return ptb_serial_forward_timed(dims, x, ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, w_qkv, w_o,
                                  w_fc1, w_fc2, y, saved, workspace, stream, nullptr);
}

int32_t ptb_serial_backward(const ptb_dims* dims, const void* dy, const void* x,
                            const void* ln1_gamma, const void* ln2_gamma, const void* w_qkv,
                            const void* w_o, const void* w_fc1, const void* w_fc2,
                            const void* saved, void* dx, void* d_ln1_gamma, void* d_ln1_beta,
                            void* d_ln2_gamma, void* d_ln2_beta, void* dw_qkv, void* dw_o,
                            void* dw_fc1, void* dw_fc2, void* workspace, void* stream) {
  return ptb_serial_backward_timed(dims, dy, x, ln1_gamma, ln2_gamma, w_qkv, w_o, w_fc1, w_fc2,
                                   saved, dx, d_ln1_gamma, d_ln1_beta, d_ln2_gamma, d_ln2_beta,
                                   dw_qkv, dw_o, dw_fc1, dw_fc2, workspace, stream, nullptr);
}

int32_t ptb_lamb_workspace_bytes(const ptb_lamb_tensor* tensors, int32_t n, size_t* bytes) {
  if (tensors == nullptr || bytes == nullptr) return PTB_ERR_NULL;
  if (n < 1 || n > PTB_LAMB_MAX_TENSORS) return PTB_ERR_ARG;
  size_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t ne = tensors[i].numel;
    if (ne < 8 || ne % 8 != 0 || ne >= (int64_t(1) << 31)) return PTB_ERR_ARG;
    blocks += static_cast<size_t>(ptb::lamb_blocks(ne));
  }
  *bytes = align_up(blocks * 2 * sizeof(double));
  return PTB_OK;
}

namespace {
// Checks of one LAMB call (everything but the scratch); fills the kernels'
// tensor list and hyper-parameters.
int32_t lamb_args(const ptb_lamb_hyper* hyper, const ptb_lamb_tensor* tensors, int32_t n,
                  float* norms, ptb::LambTensor* ts, ptb::LambHyper* hp, size_t* scratch_bytes) {
  if (hyper == nullptr || tensors == nullptr) return PTB_ERR_NULL;
  const int32_t st = ptb_lamb_workspace_bytes(tensors, n, scratch_bytes);
  if (st != PTB_OK) return st;
  const ptb_lamb_hyper& h = *hyper;
  if (!isfinite(h.lr) || !(h.beta1 >= 0.0f && h.beta1 < 1.0f) ||
      !(h.beta2 >= 0.0f && h.beta2 < 1.0f) || !(h.eps > 0.0f) || !isfinite(h.eps) || h.step < 1)
    return PTB_ERR_ARG;
  for (int i = 0; i < n; ++i) {
    const ptb_lamb_tensor& t = tensors[i];
    const int32_t pc = check_ptrs({t.theta, t.m, t.v, t.grad, t.weight});
    if (pc != PTB_OK) return pc;
  }
  const int32_t pc = check_ptrs({norms});
  if (pc != PTB_OK) return pc;
  for (int i = 0; i < n; ++i)
    ts[i] = ptb::LambTensor{tensors[i].theta, tensors[i].m, tensors[i].v,
                            static_cast<const u16*>(tensors[i].grad),
                            static_cast<u16*>(tensors[i].weight), static_cast<long>(tensors[i].numel)};
  *hp = ptb::LambHyper{h.lr, h.beta1, h.beta2, h.eps, h.step};
  return PTB_OK;
}
}  // namespace

int32_t ptb_lamb_step(const ptb_lamb_hyper* hyper, const ptb_lamb_tensor* tensors, int32_t n,
                      float* norms, void* workspace, void* stream) {
  ptb::LambTensor ts[PTB_LAMB_MAX_TENSORS];
  ptb::LambHyper hp;
  size_t need = 0;
  int32_t st = lamb_args(hyper, tensors, n, norms, ts, &hp, &need);
  if (st != PTB_OK) return st;
  st = check_ptrs({workspace});
  if (st != PTB_OK) return st;
  PTB_HIP(ptb::launch_lamb(ts, n, hp, static_cast<double*>(workspace), norms,
                           reinterpret_cast<hipStream_t>(stream)));
  return PTB_OK;
}

int32_t ptb_lamb_step_noalloc(const ptb_lamb_hyper* hyper, const ptb_lamb_tensor* tensors,
                              int32_t n, float* norms, void* stream) {
  ptb::LambTensor ts[PTB_LAMB_MAX_TENSORS];
  ptb::LambHyper hp;
  size_t need = 0;
  const int32_t st = lamb_args(hyper, tensors, n, norms, ts, &hp, &need);
  if (st != PTB_OK) return st;
  if (need > ptb::kLambStaticScratchBytes) return PTB_ERR_SCRATCH;
  double* scratch = nullptr;  // this device's copy of the static array
  PTB_HIP(ptb::lamb_static_scratch(&scratch));
  PTB_HIP(ptb::launch_lamb(ts, n, hp, scratch, norms, reinterpret_cast<hipStream_t>(stream)));
  return PTB_OK;
}

int32_t ptb_dropout_mask(uint64_t seed, uint32_t stream, float p, int64_t n, void* mask,
                         void* stream_handle) {
  if (!(p >= 0.0f && p < 1.0f) || n < 0 || n >= (int64_t(1) << 32) - 4) return PTB_ERR_ARG;
  if (mask == nullptr) return PTB_ERR_NULL;
  ptb_dims d{};
  d.dropout_p = p;
  d.dropout_seed = seed;
  ptb::Dropout dr = dropout_of(d, 0);
  dr.stream = stream;
  if (!dr.on) {  // p = 0: every element kept
    dr.on = 1;
    dr.t = 0;
    dr.k0 = static_cast<uint32_t>(seed & 0xffffffffu);
    dr.k1 = static_cast<uint32_t>(seed >> 32);
  }
  PTB_HIP(ptb::launch_dropout_mask(static_cast<uint8_t*>(mask), n, dr,
                                   reinterpret_cast<hipStream_t>(stream_handle)));
  return PTB_OK;
}

// ---- FP8 GEMM variant

int32_t ptb_fp8_weights_bytes(const ptb_dims* dims, int32_t recipe, size_t* bytes) {
  Shape s;
  const int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = fp8_weight_layout(s, recipe == PTB_FP8_MX).total;
  return PTB_OK;
}

int32_t ptb_fp8_saved_bytes(const ptb_dims* dims, int32_t recipe, size_t* bytes) {
  Shape s;
  const int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = fp8_saved_layout(s, recipe == PTB_FP8_MX).total;
  return PTB_OK;
}

int32_t ptb_fp8_workspace_bytes(const ptb_dims* dims, int32_t recipe, size_t* bytes) {
  Shape s;
  const int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  if (bytes == nullptr) return PTB_ERR_NULL;
  *bytes = fp8_work_layout(s, recipe == PTB_FP8_MX).total;
  return PTB_OK;
}

int32_t ptb_fp8_weights_layout(const ptb_dims* dims, int32_t recipe, size_t* offsets) {
  Shape s;
  const int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  if (offsets == nullptr) return PTB_ERR_NULL;
  const Fp8WeightLayout L = fp8_weight_layout(s, recipe == PTB_FP8_MX);
  offsets[PTB_FP8_AMAX] = L.amax;
  offsets[PTB_FP8_W1T] = L.w1t.codes;
  offsets[PTB_FP8_W1] = L.w1r.codes;
  offsets[PTB_FP8_W2T] = L.w2t.codes;
  offsets[PTB_FP8_W2] = L.w2r.codes;
  offsets[PTB_FP8_W1T_S] = L.w1t.scales;
  offsets[PTB_FP8_W1_S] = L.w1r.scales;
  offsets[PTB_FP8_W2T_S] = L.w2t.scales;
  offsets[PTB_FP8_W2_S] = L.w2r.scales;
  return PTB_OK;
}

int32_t ptb_fp8_quantize(const void* x, int32_t rows, int32_t cols, int32_t format, float* amax,
                         void* q, void* qt, void* stream) {
  if (x == nullptr || amax == nullptr || (q == nullptr && qt == nullptr)) return PTB_ERR_NULL;
  if ((format != PTB_FP8_E4M3 && format != PTB_FP8_E5M2)) return PTB_ERR_ARG;
  if (rows < 1 || cols < 8 || cols % 8 != 0 || static_cast<long>(rows) * cols >= (1L << 30))
    return PTB_ERR_DIMS;
  if (!aligned16(x) || !aligned16(amax) || (q != nullptr && !aligned16(q)) ||
      (qt != nullptr && !aligned16(qt)))
    return PTB_ERR_ALIGN;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const size_t ldq = pad64(static_cast<size_t>(cols));
  const size_t ldqt = pad64(static_cast<size_t>(rows));
  PTB_HIP(ptb::launch_zero_i32(reinterpret_cast<int*>(amax), 1, strm));
  PTB_HIP(cast_fp8(cast_one(x, cols, rows, cols),
                   format == PTB_FP8_E4M3 ? ptb::FP8_E4M3 : ptb::FP8_E5M2, amax,
                   static_cast<uint8_t*>(q), ldq, static_cast<uint8_t*>(qt), ldqt, strm));
  return PTB_OK;
}

int32_t ptb_fp8_quantize_mx(const void* x, int32_t rows, int32_t cols, int32_t format, void* q,
                            void* q_scales, void* qt, void* qt_scales, void* stream) {
  const bool row_copy = q != nullptr && q_scales != nullptr;
  const bool col_copy = qt != nullptr && qt_scales != nullptr;
  if (x == nullptr || (!row_copy && !col_copy)) return PTB_ERR_NULL;
  if ((format != PTB_FP8_E4M3 && format != PTB_FP8_E5M2)) return PTB_ERR_ARG;
  if (rows < 1 || cols < 8 || cols % 8 != 0 || static_cast<long>(rows) * cols >= (1L << 30))
    return PTB_ERR_DIMS;
  if (!aligned16(x) || (row_copy && (!aligned16(q) || !aligned16(q_scales))) ||
      (col_copy && (!aligned16(qt) || !aligned16(qt_scales))))
    return PTB_ERR_ALIGN;
  const size_t R = static_cast<size_t>(rows), C = static_cast<size_t>(cols);
  PTB_HIP(ptb::launch_cast_mx(
      cast_one(x, cols, rows, cols), format == PTB_FP8_E4M3 ? ptb::FP8_E4M3 : ptb::FP8_E5M2,
      row_copy ? static_cast<uint8_t*>(q) : nullptr, static_cast<int>(pad128(C)),
      row_copy ? static_cast<uint32_t*>(q_scales) : nullptr, static_cast<int>(pad128(R)),
      col_copy ? static_cast<uint8_t*>(qt) : nullptr, static_cast<int>(pad128(R)),
      col_copy ? static_cast<uint32_t*>(qt_scales) : nullptr, static_cast<int>(pad128(C)),
      reinterpret_cast<hipStream_t>(stream)));
  return PTB_OK;
}


int32_t ptb_fp8_cast_weights(const ptb_dims* dims, int32_t recipe, const void* w_qkv,
                             const void* w_o, const void* w_fc1, const void* w_fc2,
                             void* fp8_weights, void* stream) {
  Shape s;
  int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({w_qkv, w_o, w_fc1, w_fc2, fp8_weights});
  if (st != PTB_OK) return st;
  const bool mx = recipe == PTB_FP8_MX;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const Fp8WeightLayout L = fp8_weight_layout(s, mx);
  float* amax = mx ? nullptr : at<float>(fp8_weights, L.amax);
  if (!mx) PTB_HIP(ptb::launch_zero_i32(reinterpret_cast<int*>(amax), 2, strm));
  // W1 = [W_qkv | W_fc1] [h, N1]: row-wise for the dgrad, transposed for the forward
  PTB_HIP(cast_copies(mx, cast_two(w_qkv, 3 * s.hl, w_fc1, s.f, 3 * s.hl, 0, s.h, s.N1),
                      ptb::FP8_E4M3, amax, copy_at(fp8_weights, L.w1r),
                      copy_at(fp8_weights, L.w1t), strm));
  // W2 = [W_o ; W_fc2] [K2, h]
  PTB_HIP(cast_copies(mx, cast_two(w_o, s.h, w_fc2, s.h, s.hl, 1, s.K2, s.h), ptb::FP8_E4M3,
                      mx ? nullptr : amax + 1, copy_at(fp8_weights, L.w2r),
                      copy_at(fp8_weights, L.w2t), strm));
  return PTB_OK;
}

int32_t ptb_fp8_forward(const ptb_dims* dims, int32_t recipe, const void* x,
                        const void* ln_gamma, const void* ln_beta, const void* fp8_weights,
                        void* y, void* saved, void* workspace, void* stream,
                        void* const* ev) {
  Shape s;
  int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({x, ln_gamma, ln_beta, fp8_weights, y, saved, workspace});
  if (st != PTB_OK) return st;
  const bool mx = recipe == PTB_FP8_MX;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const Fp8SavedLayout SL = fp8_saved_layout(s, mx);
  const SavedLayout& L = SL.base;
  const Fp8WorkLayout W = fp8_work_layout(s, mx);
  const Fp8WeightLayout WL = fp8_weight_layout(s, mx);
  const ptb::GemmScratch gs{at<float>(workspace, W.base.gemm_partials),
                            at<int>(workspace, W.base.counters), W.base.max_tiles};
  u16* a = at<u16>(saved, L.off[PTB_SAVED_A]);
  float* mu = at<float>(saved, L.off[PTB_SAVED_MU]);
  float* rstd = at<float>(saved, L.off[PTB_SAVED_RSTD]);
  u16* qkv = at<u16>(saved, L.off[PTB_SAVED_QKV]);
  u16* u = at<u16>(saved, L.off[PTB_SAVED_U]);
  u16* g = at<u16>(saved, L.off[PTB_SAVED_G]);
  u16* c = at<u16>(saved, L.off[PTB_SAVED_C]);
  float* lse = at<float>(saved, L.off[PTB_SAVED_LSE]);
  u16* qk16 = at<u16>(saved, L.off[PTB_SAVED_QK16]);
  float* samax = at<float>(saved, SL.amax);  // [0] a, [1] [c | g] (current scaling)
  const float* wamax = mx ? nullptr : at<float>(fp8_weights, WL.amax);

  PTB_HIP(ptb::launch_zero_i32(reinterpret_cast<int*>(samax), 2, strm));
  // the LayerNorm launch also clears the arrival counters of the launches after it
  PTB_STAGE(0, ptb::launch_layernorm_fwd(static_cast<const u16*>(x),
                                    static_cast<const u16*>(ln_gamma),
                                    static_cast<const u16*>(ln_beta), a, nullptr, mu, rstd,
                                    static_cast<int>(s.T), static_cast<int>(s.h), dims->ln_eps,
                                    strm, s.rms, gs.counters, gs.max_tiles));
  // a row-wise for the [QKV | FC1] product, transposed (stashed) for its
  // weight gradient
  PTB_STAGE(1, cast_copies(mx, cast_one(a, s.h, s.T, s.h), ptb::FP8_E4M3, samax,
                           copy_at(workspace, W.a8), copy_at(saved, SL.a8t), strm));
  {  // [qkv | u] = a W1 in one FP8 product; q, k stored as value + residual, g = GeLU(u)
    ptb::GemmProblem pr;
    pr.epi = ptb::Epilogue{};
    pr.epi.o0 = qkv; pr.epi.ld0 = static_cast<int>(3 * s.hl);
    pr.epi.o1 = u; pr.epi.o2 = g; pr.epi.ld1 = static_cast<int>(s.f);
    pr.epi.ld2 = static_cast<int>(s.f);
    pr.epi.o3 = qk16; pr.epi.ld3 = static_cast<int>(2 * s.hl);
    pr.epi.lo_cols = static_cast<int>(2 * s.hl);
    pr.epi.split = static_cast<int>(3 * s.hl);
    PTB_STAGE(2, gemm8(mx, pr, copy_at(workspace, W.a8), ptb::FP8_E4M3, samax,
                       copy_at(fp8_weights, WL.w1t), ptb::FP8_E4M3, wamax, ptb::EPI_QKV_GELU,
                       gs, strm));
  }
  const ptb::AttnScratch as{gs.partials, ptb::kGemmPartialBytes / sizeof(float), gs.counters,
                            gs.max_tiles, ptb::device_compute_units()};
  PTB_STAGE(3, ptb::launch_attention_fwd(qkv, qk16, c, lse, static_cast<int>(s.b),
                                    static_cast<int>(s.s), static_cast<int>(s.n),
                                    static_cast<int>(s.d), static_cast<int>(s.w), as, strm));
  PTB_STAGE(4, cast_copies(mx, cast_two(c, s.hl, g, s.f, s.hl, 0, s.T, s.K2), ptb::FP8_E4M3,
                           samax + 1, copy_at(workspace, W.cg8), copy_at(saved, SL.cg8t), strm));
  {  // y = x + [c | g] W2
    ptb::GemmProblem pr;
    pr.epi = ptb::Epilogue{};
    pr.epi.o0 = static_cast<u16*>(y); pr.epi.i0 = static_cast<const u16*>(x);
    pr.epi.ld0 = static_cast<int>(s.h);
    PTB_STAGE(5, gemm8(mx, pr, copy_at(workspace, W.cg8), ptb::FP8_E4M3, samax + 1,
                       copy_at(fp8_weights, WL.w2t), ptb::FP8_E4M3, mx ? nullptr : wamax + 1,
                       ptb::EPI_RESIDUAL, gs, strm));
  }
  return PTB_OK;
}

int32_t ptb_fp8_backward(const ptb_dims* dims, int32_t recipe, const void* dy,
                         const void* x, const void* ln_gamma, const void* fp8_weights,
                         const void* saved, void* dx, void* d_ln_gamma, void* d_ln_beta,
                         void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2, void* workspace,
                         void* stream, void* const* ev) {
  Shape s;
  int32_t st = check_fp8_dims(dims, recipe, &s);
  if (st != PTB_OK) return st;
  st = check_ptrs({dy, x, ln_gamma, fp8_weights, saved, dx, d_ln_gamma, d_ln_beta, dw_qkv, dw_o,
                   dw_fc1, dw_fc2, workspace});
  if (st != PTB_OK) return st;
  const bool mx = recipe == PTB_FP8_MX;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const Fp8SavedLayout SL = fp8_saved_layout(s, mx);
  const SavedLayout& L = SL.base;
  const Fp8WorkLayout W = fp8_work_layout(s, mx);
  const Fp8WeightLayout WL = fp8_weight_layout(s, mx);
  const float* mu = at<float>(saved, L.off[PTB_SAVED_MU]);
  const float* rstd = at<float>(saved, L.off[PTB_SAVED_RSTD]);
  const u16* qkv = at<u16>(saved, L.off[PTB_SAVED_QKV]);
  const u16* u = at<u16>(saved, L.off[PTB_SAVED_U]);
  const u16* c = at<u16>(saved, L.off[PTB_SAVED_C]);
  const float* lse = at<float>(saved, L.off[PTB_SAVED_LSE]);
  const u16* qk16 = at<u16>(saved, L.off[PTB_SAVED_QK16]);
  u16* dc = at<u16>(workspace, W.base.dc);
  u16* dz = at<u16>(workspace, W.base.dz);
  u16* da = at<u16>(workspace, W.base.da);
  float* delta = at<float>(workspace, W.base.delta);
  float* partials = at<float>(workspace, W.base.partials);
  const ptb::GemmScratch gs{at<float>(workspace, W.base.gemm_partials),
                            at<int>(workspace, W.base.counters), W.base.max_tiles};
  float* amax = at<float>(workspace, W.amax);
  const float* samax = at<float>(saved, SL.amax);  // the forward's: [0] a, [1] [c | g]
  const float* wamax = mx ? nullptr : at<float>(fp8_weights, WL.amax);
  const u16* DY = static_cast<const u16*>(dy);
  const int T = static_cast<int>(s.T), h = static_cast<int>(s.h);

  PTB_HIP(ptb::launch_zero_i32(gs.counters, gs.max_tiles, strm));
  PTB_HIP(ptb::launch_zero_i32(reinterpret_cast<int*>(amax), AMAX_COUNT, strm));
  PTB_STAGE(0, cast_copies(mx, cast_one(DY, s.h, s.T, s.h), ptb::FP8_E5M2, amax + AMAX_DY,
                           copy_at(workspace, W.dy8), copy_at(workspace, W.dy8t), strm));
  {  // dgrad through [O ; FC2]: dc, and du = dg * GeLU'(u) into dZ's FC1 columns
    ptb::GemmProblem pr;
    pr.epi = ptb::Epilogue{};
    pr.epi.o0 = dc; pr.epi.ld0 = static_cast<int>(s.hl);
    pr.epi.o1 = dz; pr.epi.ld1 = static_cast<int>(s.N1);
    pr.epi.col_off1 = static_cast<int>(3 * s.hl);
    pr.epi.i0 = u; pr.epi.ld2 = static_cast<int>(s.f);
    pr.epi.split = static_cast<int>(s.hl);
    PTB_STAGE(1, gemm8(mx, pr, copy_at(workspace, W.dy8), ptb::FP8_E5M2, amax + AMAX_DY,
                       copy_at(fp8_weights, WL.w2r), ptb::FP8_E4M3, mx ? nullptr : wamax + 1,
                       ptb::EPI_DGELU, gs, strm));
  }
  const ptb::AttnScratch as{gs.partials, ptb::kGemmPartialBytes / sizeof(float), gs.counters,
                            gs.max_tiles, ptb::device_compute_units()};
  PTB_STAGE(2, ptb::launch_attention_bwd(qkv, qk16, c, lse, dc, delta, dz, static_cast<int>(s.N1),
                                    static_cast<int>(s.b), static_cast<int>(s.s),
                                    static_cast<int>(s.n), static_cast<int>(s.d),
                                    static_cast<int>(s.w), as, strm));
  {  // wgrad of [O ; FC2]: [c | g]^T dy
    ptb::GemmProblem pr;
    pr.epi = ptb::Epilogue{};
    pr.epi.o0 = static_cast<u16*>(dw_o); pr.epi.ld0 = h;
    pr.epi.o1 = static_cast<u16*>(dw_fc2); pr.epi.ld1 = h;
    pr.epi.split = static_cast<int>(s.hl);
    PTB_STAGE(3, gemm8(mx, pr, copy_at(saved, SL.cg8t), ptb::FP8_E4M3, samax + 1,
                       copy_at(workspace, W.dy8t), ptb::FP8_E5M2, amax + AMAX_DY,
                       ptb::EPI_STORE2_ROWS, gs, strm));
  }
  PTB_STAGE(4, cast_copies(mx, cast_one(dz, s.N1, s.T, s.N1), ptb::FP8_E5M2, amax + AMAX_DZ,
                           copy_at(workspace, W.dz8), copy_at(workspace, W.dz8t), strm));
  {  // dgrad through [QKV | FC1]: da = dZ W1^T
    ptb::GemmProblem pr;
    pr.epi = ptb::Epilogue{};
    pr.epi.o0 = da; pr.epi.ld0 = h;
    pr.epi.split = h;  // one output
    PTB_STAGE(5, gemm8(mx, pr, copy_at(workspace, W.dz8), ptb::FP8_E5M2, amax + AMAX_DZ,
                       copy_at(fp8_weights, WL.w1r), ptb::FP8_E4M3, wamax,
                       ptb::EPI_STORE2_COLS, gs, strm));
  }
  {  // wgrad of [QKV | FC1]: a^T dZ
    ptb::GemmProblem pr;
    pr.epi = ptb::Epilogue{};
    pr.epi.o0 = static_cast<u16*>(dw_qkv); pr.epi.ld0 = static_cast<int>(3 * s.hl);
    pr.epi.o1 = static_cast<u16*>(dw_fc1); pr.epi.ld1 = static_cast<int>(s.f);
    pr.epi.split = static_cast<int>(3 * s.hl);
    PTB_STAGE(6, gemm8(mx, pr, copy_at(saved, SL.a8t), ptb::FP8_E4M3, samax,
                       copy_at(workspace, W.dz8t), ptb::FP8_E5M2, amax + AMAX_DZ,
                       ptb::EPI_STORE2_COLS, gs, strm));
  }
  PTB_STAGE(7, ptb::launch_layernorm_bwd(da, static_cast<const u16*>(x),
                                    static_cast<const u16*>(ln_gamma), mu, rstd, DY,
                                    static_cast<u16*>(dx), partials,
                                    static_cast<u16*>(d_ln_gamma), static_cast<u16*>(d_ln_beta),
                                    T, h, strm, s.rms));
  return PTB_OK;
}

}  // extern "C"
