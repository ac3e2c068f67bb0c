// Drives every entry point of the C ABI (include/ptb.h) on host buffers sized
// by the library's own size queries, over shapes that exercise the layout and
// plan arithmetic (ragged sizes, d = 64 and 128, single tokens, windows above
// the sequence, the variants, dropout, both FP8 recipes, wide layers).  Built
// with the host sanitizers against the stand-in launchers of
// stub_launchers.cpp, which touch every region handed to a kernel; any
// out-of-bounds region, overflow or undefined behaviour in the host code
// aborts the run.  Exit status 0 and "ok" on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "ptb.h"

namespace {

struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    p = aligned_alloc(256, (bytes + 255) / 256 * 256);
    memset(p, 0, (bytes + 255) / 256 * 256);
  }
  ~Buf() { free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

int failures = 0;
void expect(int32_t st, int32_t want, const char* what) {
  if (st != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, st, ptb_status_string(st), want);
    ++failures;
  }
}

size_t query(int32_t (*f)(const ptb_dims*, size_t*), const ptb_dims& d) {
  size_t n = 0;
  expect(f(&d, &n), PTB_OK, "size query");
  return n;
}
size_t query8(int32_t (*f)(const ptb_dims*, int32_t, size_t*), const ptb_dims& d, int32_t r) {
  size_t n = 0;
  expect(f(&d, r, &n), PTB_OK, "fp8 size query");
  return n;
}

void run_layer(const ptb_dims& d) {
  const size_t T = static_cast<size_t>(d.batch) * d.seq, h = d.hidden;
  const size_t hl = static_cast<size_t>(d.heads) * d.head_dim, f = d.ffn;
  const size_t f1 = d.mlp == PTB_MLP_SWIGLU ? 2 * f : f;
  Buf x(T * h * 2), y(T * h * 2), dy(T * h * 2), dx(T * h * 2);
  Buf g1(h * 2), b1(h * 2), g2(h * 2), b2(h * 2), dg1(h * 2), db1(h * 2), dg2(h * 2), db2(h * 2);
  Buf wqkv(h * 3 * hl * 2), wo(hl * h * 2), w1(h * f1 * 2), w2(f * h * 2);
  Buf dwqkv(h * 3 * hl * 2), dwo(hl * h * 2), dw1(h * f1 * 2), dw2(f * h * 2);
  {
#ifdef PLANT_SHORT_SAVED  // the harness's own check: a stash 4 KB short must be caught
    Buf saved(query(ptb_saved_bytes, d) - 4096), work(query(ptb_workspace_bytes, d));
#else
    Buf saved(query(ptb_saved_bytes, d)), work(query(ptb_workspace_bytes, d));
#endif
    expect(ptb_forward(&d, x.p, g1.p, b1.p, wqkv.p, wo.p, w1.p, w2.p, y.p, saved.p, work.p,
                       nullptr), PTB_OK, "ptb_forward");
    expect(ptb_backward(&d, dy.p, x.p, g1.p, wqkv.p, wo.p, w1.p, w2.p, saved.p, dx.p, dg1.p,
                        db1.p, dwqkv.p, dwo.p, dw1.p, dw2.p, work.p, nullptr), PTB_OK,
           "ptb_backward");
    std::vector<size_t> off(PTB_SAVED_COUNT);
    expect(ptb_saved_layout(&d, off.data()), PTB_OK, "ptb_saved_layout");
  }
  {
    Buf saved(query(ptb_serial_saved_bytes, d)), work(query(ptb_serial_workspace_bytes, d));
    expect(ptb_serial_forward(&d, x.p, g1.p, b1.p, g2.p, b2.p, wqkv.p, wo.p, w1.p, w2.p, y.p,
                              saved.p, work.p, nullptr), PTB_OK, "ptb_serial_forward");
    expect(ptb_serial_backward(&d, dy.p, x.p, g1.p, g2.p, wqkv.p, wo.p, w1.p, w2.p, saved.p, dx.p,
                               dg1.p, db1.p, dg2.p, db2.p, dwqkv.p, dwo.p, dw1.p, dw2.p, work.p,
                               nullptr), PTB_OK, "ptb_serial_backward");
  }
  if (d.mlp == PTB_MLP_GELU && d.dropout_p == 0.0f) {
    for (int32_t r : {PTB_FP8_CURRENT, PTB_FP8_MX}) {
      Buf fw(query8(ptb_fp8_weights_bytes, d, r)), saved(query8(ptb_fp8_saved_bytes, d, r));
      Buf work(query8(ptb_fp8_workspace_bytes, d, r));
      std::vector<size_t> off(PTB_FP8_WEIGHT_PARTS);
      expect(ptb_fp8_weights_layout(&d, r, off.data()), PTB_OK, "ptb_fp8_weights_layout");
      expect(ptb_fp8_cast_weights(&d, r, wqkv.p, wo.p, w1.p, w2.p, fw.p, nullptr), PTB_OK,
             "ptb_fp8_cast_weights");
      expect(ptb_fp8_forward(&d, r, x.p, g1.p, b1.p, fw.p, y.p, saved.p, work.p, nullptr, nullptr),
             PTB_OK, "ptb_fp8_forward");
      expect(ptb_fp8_backward(&d, r, dy.p, x.p, g1.p, fw.p, saved.p, dx.p, dg1.p, db1.p, dwqkv.p,
                              dwo.p, dw1.p, dw2.p, work.p, nullptr, nullptr), PTB_OK,
             "ptb_fp8_backward");
    }
  }
}

ptb_dims dims(int b, int s, int h, int n, int dd, int f, int w, int norm = PTB_NORM_LAYERNORM,
              int mlp = PTB_MLP_GELU, float p = 0.0f) {
  ptb_dims d{};
  d.batch = b; d.seq = s; d.hidden = h; d.heads = n; d.head_dim = dd; d.ffn = f; d.window = w;
  d.ln_eps = 1e-5f; d.norm = norm; d.mlp = mlp; d.dropout_p = p; d.dropout_layer = 3;
  d.dropout_seed = 0x123456789abcdef0ull;
  return d;
}

void run_quantize() {
  for (int rc : {0, 1}) {
    const int rows = rc ? 130 : 3, cols = rc ? 264 : 200;
    Buf x(static_cast<size_t>(rows) * cols * 2), amax(4);
    const size_t p64r = (rows + 63) / 64 * 64, p64c = (cols + 63) / 64 * 64;
    Buf q(static_cast<size_t>(rows) * p64c), qt(static_cast<size_t>(cols) * p64r);
    expect(ptb_fp8_quantize(x.p, rows, cols, PTB_FP8_E4M3, static_cast<float*>(amax.p), q.p,
                            qt.p, nullptr), PTB_OK, "ptb_fp8_quantize");
    const size_t p128r = (rows + 127) / 128 * 128, p128c = (cols + 127) / 128 * 128;
    Buf mq(rows * p128c), mqs(p128c / 128 * p128r * 4), mqt(cols * p128r),
        mqts(p128r / 128 * p128c * 4);
    expect(ptb_fp8_quantize_mx(x.p, rows, cols, PTB_FP8_E5M2, mq.p, mqs.p, mqt.p, mqts.p, nullptr),
           PTB_OK, "ptb_fp8_quantize_mx");
  }
}

void run_lamb_and_dropout() {
  const int64_t sizes[] = {64, 16384, 16384 * 3 + 8, 100000};
  std::vector<Buf*> bufs;
  std::vector<ptb_lamb_tensor> ts;
  for (int64_t ne : sizes) {
    Buf* th = new Buf(ne * 4); Buf* m = new Buf(ne * 4); Buf* v = new Buf(ne * 4);
    Buf* g = new Buf(ne * 2); Buf* w = new Buf(ne * 2);
    bufs.insert(bufs.end(), {th, m, v, g, w});
    ts.push_back(ptb_lamb_tensor{static_cast<float*>(th->p), static_cast<float*>(m->p),
                                 static_cast<float*>(v->p), g->p, w->p, ne});
  }
  size_t wb = 0;
  expect(ptb_lamb_workspace_bytes(ts.data(), static_cast<int32_t>(ts.size()), &wb), PTB_OK,
         "ptb_lamb_workspace_bytes");
  Buf work(wb), norms(ts.size() * 8);
  ptb_lamb_hyper hp{1e-3f, 0.9f, 0.999f, 1e-6f, 3};
  expect(ptb_lamb_step(&hp, ts.data(), static_cast<int32_t>(ts.size()),
                       static_cast<float*>(norms.p), work.p, nullptr), PTB_OK, "ptb_lamb_step");
  expect(ptb_lamb_step_noalloc(&hp, ts.data(), static_cast<int32_t>(ts.size()),
                               static_cast<float*>(norms.p), nullptr), PTB_OK,
         "ptb_lamb_step_noalloc");
  for (Buf* b : bufs) delete b;
  for (int64_t n : {int64_t(0), int64_t(1), int64_t(1001), int64_t(65539)}) {
    Buf mask(n > 0 ? n : 1);
    expect(ptb_dropout_mask(7, 1, 0.25f, n, mask.p, nullptr), PTB_OK, "ptb_dropout_mask");
  }
}

}  // namespace

int main() {
  const ptb_dims shapes[] = {
      dims(2, 256, 256, 4, 64, 1024, 64),                 // the tiny workload
      dims(1, 200, 256, 2, 128, 320, 37),                 // ragged s, d 128
      dims(3, 97, 320, 5, 64, 448, 33),                   // ragged b, s, h, f, d 64
      dims(1, 1, 128, 1, 128, 128, 1),                    // one token
      dims(3, 2, 128, 2, 64, 128, 5),                     // two tokens per sequence
      dims(1, 131, 256, 3, 64, 320, 100000),              // window above the sequence
      dims(2, 130, 256, 2, 128, 512, 48, PTB_NORM_RMSNORM, PTB_MLP_SWIGLU),
      dims(1, 200, 256, 2, 128, 320, 37, PTB_NORM_LAYERNORM, PTB_MLP_GELU, 0.3f),  // dropout
      dims(1, 64, 4096, 32, 128, 64, 64),                 // wide layer, few tokens
      dims(2, 300, 192, 3, 64, 192, 129),                 // window just above a tile
  };
  for (const ptb_dims& d : shapes) run_layer(d);
  run_quantize();
  run_lamb_and_dropout();
  if (failures) {
    fprintf(stderr, "%d unexpected status codes\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
