// C ABI of the QLoRA linear / gated-MLP library (declared in include/qlora.h).
//
// This file validates arguments, carves the caller's workspace and enqueues
// the gfx950 kernels on the caller's stream in dependency order. It never
// allocates and never synchronizes the host.
//
// Step order follows the pages' manual autograd with rank-first bracketing
// (Mistral benchmark page, items 10-11; breakdown row "Manual Autograd MLP"):
//   linear fwd : U = X A^T  ->  Y = X W^T + s U B^T (one GEMM, LoRA as K-extension)
//   linear bwd : T = dY B, dB = s dY^T U  ->  dX = dY W + s T A (one GEMM)  ->  dA = s T^T X
//   MLP fwd    : [Ug|Uu] = X [Ag;Au]^T -> gate||up GEMM with act epilogue (g, u, H)
//                -> Ud = H Ad^T -> down GEMM
//   MLP bwd    : Td = dY Bd, dBd -> dH GEMM with act' epilogue (dg, du) -> dAd (H recomputed)
//                -> [Tg|Tu] = [dg|du] blockdiag(Bg,Bu), dBg, dBu -> dX GEMM (K = 2h) -> dAg, dAu
//   (with a bf16 weight, r <= 16 and m <= 16384, Ud and [Tg|Tu] are formed in
//   the epilogues that write H and dg, du, as per-tile partials, and only
//   summed afterwards)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qlora.h"
#include "kernels.hpp"

using namespace qlora;

namespace {

thread_local std::string g_last_error;

int hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return QLORA_EHIP;
}

#define QL_TRY(expr, where)                        \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// Bump allocator over the caller's workspace (or a size counter when base == nullptr).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

inline int64_t ceil16(int64_t x) { return (x + 15) / 16 * 16; }

// The MLP's gate and up products share one K-extension. With 2r <= 64 one
// row product forms [U_g | U_u] and the columns are
// [hi(sU_g) hi(sU_u) | lo(sU_g) lo(sU_u) | 0 ...] (ceil16(4r) wide); above
// that (r > 32) each projection has its own row product and its own
// ceil16(2r)-wide segment [hi(sU_g) lo(sU_g) 0.. | hi(sU_u) lo(sU_u) 0..].
// The same holds for [T_g | T_u] in the backward.
inline bool mlp_wide(int64_t r) { return 2 * r > 64; }
inline int64_t mlp_ke_gu(int64_t r) { return mlp_wide(r) ? 2 * ceil16(2 * r) : ceil16(4 * r); }

// the weight's absmax: the fp32 array when given, else the double-quantized form
AbsmaxSrc absmax_src(const qlora_nf4& w) {
  if (w.absmax) return AbsmaxSrc{w.absmax, nullptr, nullptr, nullptr};
  return AbsmaxSrc{nullptr, w.absmax_q, w.absmax_scale, w.absmax_offset};
}
bool bad_absmax(const AbsmaxSrc& a) { return !a.f32 && (!a.q || !a.scale || !a.offset); }
bool absmax_aligned(const AbsmaxSrc& a) {
  return ((uintptr_t)a.f32 & 3) == 0 && ((uintptr_t)a.scale & 3) == 0 && ((uintptr_t)a.offset & 3) == 0;
}
bool bad_nf4(const qlora_nf4& w) { return !w.codes || bad_absmax(absmax_src(w)); }

// Base-weight source: NF4 (codes + absmax) or, in MODE_BF16, a bf16 matrix
// used as it is (16-bit LoRA: the dequantization step becomes nothing, a copy
// or a transpose).
constexpr int MODE_BF16 = 3;
struct WSrc {
  const uint8_t* codes = nullptr;
  AbsmaxSrc amax = AbsmaxSrc{nullptr, nullptr, nullptr, nullptr};
  const uint16_t* w16 = nullptr;
  int64_t n = 0, k = 0;
};
WSrc src_nf4(const qlora_nf4& w) {
  WSrc s;
  s.codes = w.codes; s.amax = absmax_src(w); s.n = w.n; s.k = w.k;
  return s;
}
WSrc src_w16(const uint16_t* w, int64_t n, int64_t k) {
  WSrc s;
  s.w16 = w; s.n = n; s.k = k;
  return s;
}
bool bad_src(const WSrc& w, int mode) { return mode == MODE_BF16 ? !w.w16 : (!w.codes || bad_absmax(w.amax)); }

// Pointer alignment the kernels rely on (null passes: null checks are separate).
// bf16 matrices and NF4 code arrays are read and written 16 bytes at a time,
// fp32 arrays one value at a time, the bf16 LoRA gradients one value at a time.
bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool al16(const void* p) { return al(p, 16); }
bool al4(const void* p) { return al(p, 4); }
bool al2(const void* p) { return al(p, 2); }
bool src_aligned(const WSrc& w) { return al16(w.w16) && al16(w.codes) && absmax_aligned(w.amax); }

// absmax values of a weight [n][k]
inline int64_t absmax_count(const WSrc& w) { return w.n * (w.k / 64); }

// The fused-dequant GEMM reads fp32 absmax: the stored array, or the
// double-quantized one decoded into `buf` (absmax_count floats of workspace).
hipError_t fused_absmax(const WSrc& w, float* buf, hipStream_t st, const float** out) {
  if (w.amax.f32) {
    *out = w.amax.f32;
    return hipSuccess;
  }
  *out = buf;
  return launch_absmax_dq_dequant(w.amax.q, w.amax.scale, w.amax.offset, absmax_count(w), buf, st);
}
// a bf16 copy of the weight (or of its transpose) lives in the workspace
bool staged_like(int mode) { return mode == QLORA_DEQUANT_STAGED || mode == MODE_BF16; }

// The MLP's two row products over h-wide activations (Ud = H Ad^T and
// [Tg | Tu] = [dg | du] blockdiag(Bg, Bu)) come from the epilogues of the
// GEMMs that write those activations (any weight source) when r <= 16 and
// m <= 16384; otherwise a separate pass reads the activations back. Measured
// on the Llama-7B MLP, the epilogue form gains 1.2% at 8192 tokens, breaks
// even at 16384 and loses 1-2% from 24576 tokens up.
bool rp_epilogue(int64_t r, int64_t m) { return r <= 16 && m <= 16384; }

// QLORA_DEQUANT_AUTO: fused up to 1024 tokens, staged above. Measured on the
// Llama-7B MLP fwd+bwd: fused is 9% faster at 1024 tokens (no dequant passes
// to amortize), 3% slower at 2048 and 16% slower at 8192 (each workgroup
// dequantizes its B tiles again, where staged dequantizes each weight once).
constexpr int64_t kAutoFusedMaxTokens = 1024;
// the MLP backward's dBg, dBu reductions: one launch up to this many tokens
constexpr int64_t kMergedDbTokens = 4096;
int resolve_mode(int mode, int64_t m) {
  if (mode == QLORA_DEQUANT_AUTO) return m <= kAutoFusedMaxTokens ? QLORA_DEQUANT_FUSED : QLORA_DEQUANT_STAGED;
  return mode;
}

bool valid_mode(int mode) { return mode >= QLORA_DEQUANT_AUTO && mode <= QLORA_DEQUANT_STAGED; }

// Split-K partials of a store GEMM (M x N, depth K): the launch gives a small
// output several K ranges when it has too few tiles to fill the chip (bf16 or
// NF4 B operand alike).
int64_t splitk_elems(int64_t M, int64_t N, int64_t K) {
  if (M <= 0) return 0;
  const int sp = gemm_splits((int)M, (int)N, (int)K);
  return sp > 1 ? sp * M * N : 0;
}
void use_splitk(GemmArgs& g, float* part) {
  const int sp = gemm_splits(g.M, g.N, g.K);
  if (sp > 1) { g.splits = sp; g.part = part; }
}

// ------------------------------------------------------------ linear plan --
struct LinearFwdWs {
  uint16_t* bext;  // [n][KE]
  uint16_t* uext;  // [m][KE]
  uint16_t* wbf;   // [n][k] (staged)
  float* rpart;    // row-product split partials
  float* kpart;    // split-K partials of the GEMM
  float* amx;      // fused: fp32 absmax decoded from a double-quantized weight
};

size_t plan_linear_fwd(Carver& c, int64_t m, int64_t k, int64_t n, int64_t r, int mode, LinearFwdWs* w) {
  const int64_t KE = ceil16(2 * r);
  LinearFwdWs t;
  t.bext = c.take<uint16_t>(n * KE);
  t.uext = c.take<uint16_t>(m * KE);
  t.wbf = mode == QLORA_DEQUANT_STAGED ? c.take<uint16_t>(n * k) : nullptr;
  t.rpart = c.take<float>(16 * m * r);
  t.kpart = c.take<float>(splitk_elems(m, n, k));
  t.amx = c.take<float>(mode == QLORA_DEQUANT_FUSED ? n * (k / 64) : 0);
  if (w) *w = t;
  return c.off;
}

struct LinearBwdWs {
  uint16_t* lt;    // [r][n]   B^T
  uint16_t* bext;  // [k][KE]  [A^T | A^T]
  float* t;        // [m][r]
  uint16_t* text;  // [m][KE]
  float* part;     // [chunks][max(n,k)][r]
  uint16_t* wt;    // [k][n]   dequantized W^T
  float* rpart;    // row-product split partials
  float* kpart;    // split-K partials of the dX GEMM
  float* amx;      // fused: fp32 absmax decoded from a double-quantized weight
};

size_t plan_linear_bwd(Carver& c, int64_t m, int64_t k, int64_t n, int64_t r, int mode, LinearBwdWs* w) {
  const int64_t KE = ceil16(2 * r);
  const int64_t chunks = colreduce_chunks((int)std::max<int64_t>(m, 1));
  LinearBwdWs t;
  t.lt = c.take<uint16_t>(r * n);
  t.bext = c.take<uint16_t>(k * KE);
  t.t = c.take<float>(m * r);
  t.text = c.take<uint16_t>(m * KE);
  t.part = c.take<float>(chunks * (n + k) * r);   // dB and dA partial sets side by side
  t.wt = staged_like(mode) ? c.take<uint16_t>(k * n) : nullptr;
  t.rpart = c.take<float>(16 * m * r);
  t.kpart = c.take<float>(splitk_elems(m, k, n));
  t.amx = c.take<float>(mode == QLORA_DEQUANT_FUSED ? n * (k / 64) : 0);
  if (w) *w = t;
  return c.off;
}

// --------------------------------------------------------------- MLP plan --
struct MlpFwdWs {
  uint16_t* lgu;     // [2r][d]
  uint16_t* bextgu;  // [2h][KEgu]
  uint16_t* bextd;   // [d][KEd]
  uint16_t* uextgu;  // [m][KEgu]
  uint16_t* uextd;   // [m][KEd]
  uint16_t* H;       // [m][h]
  uint16_t* wgu;     // [2h][d] staged, 32-row interleave of gate/up
  uint16_t* wd;      // [d][h]  staged
  float* rpart;      // row-product split partials
  float* kpart;      // split-K partials of the down GEMM
  float* amx;        // fused: fp32 absmax of gate, up, down decoded from a
                     // double-quantized form ([h][d/64], [h][d/64], [d][h/64])
};

size_t plan_mlp_fwd(Carver& c, int64_t m, int64_t d, int64_t h, int64_t r, int mode, MlpFwdWs* w) {
  const int64_t KEgu = mlp_ke_gu(r), KEd = ceil16(2 * r);
  MlpFwdWs t;
  t.lgu = c.take<uint16_t>(2 * r * d);
  t.bextgu = c.take<uint16_t>(2 * h * KEgu);
  t.bextd = c.take<uint16_t>(d * KEd);
  t.uextgu = c.take<uint16_t>(m * KEgu);
  t.uextd = c.take<uint16_t>(m * KEd);
  t.H = c.take<uint16_t>(m * h);
  t.wgu = staged_like(mode) ? c.take<uint16_t>(2 * h * d) : nullptr;
  t.wd = mode == QLORA_DEQUANT_STAGED ? c.take<uint16_t>(d * h) : nullptr;
  t.rpart = c.take<float>(std::max<int64_t>(16 * 2 * r, rp_epilogue(r, m) ? gemm_rowprod_splits((int)(2 * h)) * r : 0) * m);
  t.kpart = c.take<float>(splitk_elems(m, d, h));
  t.amx = c.take<float>(mode == QLORA_DEQUANT_FUSED ? 3 * h * (d / 64) : 0);
  if (w) *w = t;
  return c.off;
}

struct MlpBwdWs {
  uint16_t* ltd;     // [r][d]     Bd^T
  uint16_t* bextdh;  // [h][KEd]   [Ad^T | Ad^T]
  uint16_t* ltgu;    // [2r][2h]   blockdiag(Bg^T, Bu^T)
  uint16_t* bextdx;  // [d][KEgu]  [Ag^T | Au^T | Ag^T | Au^T]
  float* td;         // [m][r]
  uint16_t* textd;   // [m][KEd]
  uint16_t* dgu;     // [m][2h]
  float* tgu;        // [m][2r]
  uint16_t* textgu;  // [m][KEgu]
  float* part;       // [chunks][max(d,h)][2r]
  uint16_t* wdt;     // [h][d]
  uint16_t* wgut;    // [d][2h]
  float* rpart;      // row-product split partials
  float* kpart;      // split-K partials of the dX GEMM
  float* amx;        // fused: decoded fp32 absmax of gate, up, down (as forward)
};

size_t plan_mlp_bwd(Carver& c, int64_t m, int64_t d, int64_t h, int64_t r, int mode, MlpBwdWs* w) {
  const int64_t KEgu = mlp_ke_gu(r), KEd = ceil16(2 * r);
  const int64_t chunks = colreduce_chunks((int)std::max<int64_t>(m, 1));
  MlpBwdWs t;
  t.ltd = c.take<uint16_t>(r * d);
  t.bextdh = c.take<uint16_t>(h * KEd);
  t.ltgu = c.take<uint16_t>(2 * r * 2 * h);
  t.bextdx = c.take<uint16_t>(d * KEgu);
  t.td = c.take<float>(m * r);
  t.textd = c.take<uint16_t>(m * KEd);
  t.dgu = c.take<uint16_t>(m * 2 * h);
  t.tgu = c.take<float>(m * 2 * r);
  t.textgu = c.take<uint16_t>(m * KEgu);
  t.part = c.take<float>(chunks * std::max(d, h) * 2 * r);
  t.wdt = staged_like(mode) ? c.take<uint16_t>(h * d) : nullptr;
  t.wgut = staged_like(mode) ? c.take<uint16_t>(d * 2 * h) : nullptr;
  t.rpart = c.take<float>(std::max<int64_t>(16, rp_epilogue(r, m) ? gemm_rowprod_splits((int)h) : 0) * 2 * r * m);
  t.kpart = c.take<float>(splitk_elems(m, d, 2 * h));
  t.amx = c.take<float>(mode == QLORA_DEQUANT_FUSED ? 3 * h * (d / 64) : 0);
  if (w) *w = t;
  return c.off;
}

bool dims_ok(int64_t m, int64_t k, int64_t n) {
  const int64_t lim = (int64_t)1 << 30;
  return m >= 0 && k > 0 && n > 0 && k % 64 == 0 && n % 64 == 0 && m < lim && k < lim && n < lim;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need && (!ws || ws_bytes < need)) return QLORA_EWORKSPACE;
  if (ws && ((uintptr_t)ws & 255)) return QLORA_EWORKSPACE;
  return QLORA_OK;
}

GemmArgs gemm_args() {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  return a;
}

// ---- tracing: HIP events around base-GEMM launches (off by default) ----
struct TraceRec {
  hipEvent_t start, stop;
  double flops;
};
bool g_trace_on = false;
std::vector<TraceRec> g_trace;

void trace_clear() {
  for (auto& t : g_trace) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_trace.clear();
}

// Launch one base GEMM; r_alg is the LoRA rank the algorithmic count charges.
hipError_t run_gemm(const GemmArgs& g, int64_t r_alg, hipStream_t st) {
  if (!g_trace_on) return launch_gemm(g, st);
  TraceRec t;
  t.flops = 2.0 * g.M * (double)g.N * ((double)g.K + (double)r_alg);
  hipError_t e = hipEventCreate(&t.start);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&t.stop);
  if (e != hipSuccess) return e;
  e = hipEventRecord(t.start, st);
  if (e != hipSuccess) return e;
  e = launch_gemm(g, st);
  if (e != hipSuccess) return e;
  e = hipEventRecord(t.stop, st);
  if (e != hipSuccess) return e;
  g_trace.push_back(t);
  return hipSuccess;
}


// ---- helper stream: independent work of one call overlaps the big GEMMs ----
// One stream (default priority) and a few events per device, created on first
// use and kept until the process ends. A call forks work onto it with an event
// recorded on the caller's stream and joins it back before returning, so to the
// caller everything stays ordered on its own stream. The per-device mutex is
// held while a call enqueues, so events are never shared by two calls.
constexpr int kSideEvents = 6;
struct SideCtx {
  std::mutex mu;
  bool ready = false;
  hipStream_t s = nullptr;
  hipEvent_t ev[kSideEvents];
};
constexpr int kMaxDevices = 64;
SideCtx g_side[kMaxDevices];

// Locks the device's helper context for the duration of one call.
class Side {
 public:
  explicit Side(hipStream_t main) : main_(main) {}
  ~Side() {
    if (ctx_) ctx_->mu.unlock();
  }
  hipError_t open() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ctx_ = &g_side[dev];
    ctx_->mu.lock();
    if (!ctx_->ready) {
      e = hipStreamCreateWithFlags(&ctx_->s, hipStreamNonBlocking);
      if (e != hipSuccess) return e;
      for (int i = 0; i < kSideEvents; ++i) {
        e = hipEventCreateWithFlags(&ctx_->ev[i], hipEventDisableTiming);
        if (e != hipSuccess) return e;
      }
      ctx_->ready = true;
    }
    return hipSuccess;
  }
  hipStream_t stream() const { return ctx_->s; }
  // the helper stream waits for everything enqueued so far on the caller's stream
  hipError_t fork(int i) {
    hipError_t e = hipEventRecord(ctx_->ev[i], main_);
    return e != hipSuccess ? e : hipStreamWaitEvent(ctx_->s, ctx_->ev[i], 0);
  }
  // event i marks what is enqueued so far on the helper stream ...
  hipError_t mark(int i) { return hipEventRecord(ctx_->ev[i], ctx_->s); }
  // ... and the caller's stream waits for it
  hipError_t wait(int i) { return hipStreamWaitEvent(main_, ctx_->ev[i], 0); }
  hipError_t join(int i) {
    hipError_t e = mark(i);
    return e != hipSuccess ? e : wait(i);
  }

 private:
  hipStream_t main_;
  SideCtx* ctx_ = nullptr;
};

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_EINVAL: return "invalid argument (null pointer, rank, scale, activation or mode)";
    case QLORA_ESHAPE: return "invalid shape (k, n, d, h must be positive multiples of 64; m >= 0)";
    case QLORA_EWORKSPACE: return "workspace missing, misaligned or smaller than the query's answer";
    case QLORA_EHIP: return "HIP runtime or launch error (see qlora_last_error)";
    case QLORA_ENOTIMPL: return "not implemented in this library";
  }
  return "unknown status";
}

const char* qlora_last_error(void) { return g_last_error.c_str(); }

const char* qlora_version(void) { return "qlora-mi355x 0.1 gfx950"; }

int qlora_gemm_split_count(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k < 0) return -1;
  if (m >= ((int64_t)1 << 30) || n >= ((int64_t)1 << 30) || k >= ((int64_t)1 << 30)) return 1;
  return gemm_splits((int)m, (int)n, (int)k);
}

int qlora_nf4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* absmax,
                       void* stream) {
  if (n < 0 || k < 0 || k % 64 || n >= ((int64_t)1 << 31) || k >= ((int64_t)1 << 31))
    return QLORA_ESHAPE;
  if (n * k == 0) return QLORA_OK;
  if (!w || !codes || !absmax) return QLORA_EINVAL;
  if (((uintptr_t)w & 15) || ((uintptr_t)codes & 3) || ((uintptr_t)absmax & 3)) return QLORA_ESHAPE;
  QL_TRY(launch_nf4_quantize(w, n, k, codes, absmax, (hipStream_t)stream), "nf4_quantize");
  return QLORA_OK;
}

int qlora_probe_mfma_peak(int iters, double* tflops, double* shader_ghz, void* stream) {
  if (!tflops || !shader_ghz || iters < 1) return QLORA_EINVAL;
  QL_TRY(probe_mfma_peak(iters, (hipStream_t)stream, tflops, shader_ghz), "probe_mfma_peak");
  return QLORA_OK;
}

int qlora_trace_enable(int on) {
  trace_clear();
  g_trace_on = on != 0;
  return QLORA_OK;
}

int qlora_trace_read(int64_t* launches, double* total_ms, double* total_flops) {
  if (!launches || !total_ms || !total_flops) return QLORA_EINVAL;
  double ms = 0.0, fl = 0.0;
  for (auto& t : g_trace) {
    QL_TRY(hipEventSynchronize(t.stop), "trace_read");
    float e = 0.0f;
    QL_TRY(hipEventElapsedTime(&e, t.start, t.stop), "trace_read");
    ms += e;
    fl += t.flops;
  }
  *launches = (int64_t)g_trace.size();
  *total_ms = ms;
  *total_flops = fl;
  return QLORA_OK;
}

void qlora_nf4_levels(float out_host[16]) { nf4_levels_host(out_host); }

int qlora_nf4_dequant(qlora_nf4 w, uint16_t* out, void* stream) {
  if (bad_nf4(w) || !out) return QLORA_EINVAL;
  if (!dims_ok(0, w.k, w.n)) return QLORA_ESHAPE;
  const AbsmaxSrc amax = absmax_src(w);
  if (!al16(w.codes) || !absmax_aligned(amax) || !al16(out)) return QLORA_ESHAPE;
  QL_TRY(launch_nf4_dequant_rows(w.codes, amax, w.n, w.k, out, w.k, 0, (hipStream_t)stream),
         "nf4_dequant");
  return QLORA_OK;
}

int qlora_absmax_dq_quantize(const float* absmax, int64_t nb, int8_t* q, float* scale,
                             float* offset, void* stream) {
  if (nb < 0) return QLORA_ESHAPE;
  if (nb == 0) return QLORA_OK;
  if (!absmax || !q || !scale || !offset) return QLORA_EINVAL;
  if (!al4(absmax) || !al4(scale) || !al4(offset)) return QLORA_ESHAPE;
  QL_TRY(launch_absmax_dq_quantize(absmax, nb, q, scale, offset, (hipStream_t)stream),
         "absmax_dq_quantize");
  return QLORA_OK;
}

int qlora_absmax_dq_dequant(const int8_t* q, const float* scale, const float* offset, int64_t nb,
                            float* out, void* stream) {
  if (nb < 0) return QLORA_ESHAPE;
  if (nb == 0) return QLORA_OK;
  if (!q || !scale || !offset || !out) return QLORA_EINVAL;
  if (!al4(out) || !al4(scale) || !al4(offset)) return QLORA_ESHAPE;
  QL_TRY(launch_absmax_dq_dequant(q, scale, offset, nb, out, (hipStream_t)stream), "absmax_dq_dequant");
  return QLORA_OK;
}

// ------------------------------------------------------------ linear layer --
// what the forward alone carves (the workspace query covers both directions)
static size_t linear_fwd_ws(int64_t m, int64_t k, int64_t n, int64_t r, int mode) {
  Carver a(nullptr);
  return plan_linear_fwd(a, m, k, n, r, mode, nullptr);
}

static size_t linear_ws(int64_t m, int64_t k, int64_t n, int64_t r, int mode) {
  Carver a(nullptr), b(nullptr);
  return std::max(plan_linear_fwd(a, m, k, n, r, mode, nullptr), plan_linear_bwd(b, m, k, n, r, mode, nullptr));
}

size_t qlora_linear_workspace_bytes(int64_t m, int64_t k, int64_t n, int64_t r, int mode) {
  if (!dims_ok(m, k, n) || r < 1 || r > 64 || !valid_mode(mode)) return 0;
  return linear_ws(m, k, n, r, resolve_mode(mode, m));
}

size_t qlora_linear16_workspace_bytes(int64_t m, int64_t k, int64_t n, int64_t r) {
  if (!dims_ok(m, k, n) || r < 1 || r > 64) return 0;
  return linear_ws(m, k, n, r, MODE_BF16);
}

// Argument checks of the linear forward (everything but the workspace).
static int linear_fwd_check(const uint16_t* X, int64_t m, const WSrc& w, const uint16_t* A,
                            const uint16_t* B, int64_t r, float s, uint16_t* Y, float* U_save,
                            int mode) {
  if (!A || !B || bad_src(w, mode)) return QLORA_EINVAL;
  if (m > 0 && (!X || !Y)) return QLORA_EINVAL;   // per-token tensors may be NULL when m == 0
  if (r < 1 || r > 64 || !std::isfinite(s)) return QLORA_EINVAL;
  if (!dims_ok(m, w.k, w.n)) return QLORA_ESHAPE;
  if (!src_aligned(w) || !al16(A) || !al16(B) || !al16(X) || !al16(Y) || !al4(U_save))
    return QLORA_ESHAPE;
  return QLORA_OK;
}

// mode: QLORA_DEQUANT_STAGED, QLORA_DEQUANT_FUSED or MODE_BF16 (resolved).
// traced: the base GEMM may be timed by the optional launch trace (which
// creates HIP events); the no-allocation entry point passes false.
static int linear_fwd_impl(const uint16_t* X, int64_t m, const WSrc& w, const uint16_t* A,
                           const uint16_t* B, int64_t r, float s, uint16_t* Y, float* U_save,
                           int mode, void* ws, size_t ws_bytes, void* stream, bool traced = true) {
  if (int e = linear_fwd_check(X, m, w, A, B, r, s, Y, U_save, mode)) return e;
  const int64_t k = w.k, n = w.n;
  if (int e = check_ws(ws, ws_bytes, linear_fwd_ws(m, k, n, r, mode))) return e;
  if (m == 0) return QLORA_OK;
  hipStream_t st = (hipStream_t)stream;
  Carver c(ws);
  LinearFwdWs t;
  plan_linear_fwd(c, m, k, n, r, mode, &t);
  const int KE = (int)ceil16(2 * r);

  {  // Bext = [B | B | 0]
    PrepJobs J;
    J.copy(B, r, 1, n, r, t.bext, KE, 1);
    J.copy(B, r, 1, n, r, t.bext + r, KE, 1);
    J.zero(n, KE - 2 * r, t.bext + 2 * r, KE, 1);
    QL_TRY(launch_prep(J, st), "linear_fwd: LoRA layouts");
  }
  if (mode == QLORA_DEQUANT_STAGED)
    QL_TRY(launch_nf4_dequant_rows(w.codes, w.amax, n, k, t.wbf, k, 0, st), "linear_fwd: dequant");
  QL_TRY(launch_rowdot(X, k, A, k, (int)m, (int)k, (int)r, s, U_save, nullptr, (int)r, r, t.uext,
                       KE, KE, t.rpart, st),
         "linear_fwd: U = X A^T");
  GemmArgs g = gemm_args();
  g.A = X; g.lda = k;
  if (mode == QLORA_DEQUANT_STAGED) { g.bsrc = BSRC_BF16; g.B = t.wbf; g.ldb = k; }
  else if (mode == MODE_BF16) { g.bsrc = BSRC_BF16; g.B = w.w16; g.ldb = k; }
  else {
    g.bsrc = BSRC_NF4; g.codes0 = w.codes;
    QL_TRY(fused_absmax(w, t.amx, st, &g.absmax0), "linear_fwd: absmax");
  }
  g.Ae = t.uext; g.ldae = KE; g.Be = t.bext; g.ldbe = KE;
  g.M = (int)m; g.N = (int)n; g.K = (int)k; g.KE = KE;
  g.epi = EPI_STORE; g.C = Y; g.ldc = n;
  use_splitk(g, t.kpart);
  QL_TRY(traced ? run_gemm(g, r, st) : launch_gemm(g, st), "linear_fwd: GEMM");
  return QLORA_OK;
}

static int linear_bwd_impl(const uint16_t* dY, const uint16_t* X, const float* U, int64_t m,
                           const WSrc& w, const uint16_t* A, const uint16_t* B, int64_t r, float s,
                           uint16_t* dX, uint16_t* dA, uint16_t* dB, int mode, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!A || !B || !dA || !dB || bad_src(w, mode)) return QLORA_EINVAL;
  if (m > 0 && (!dY || !X || !U)) return QLORA_EINVAL;   // may be NULL when m == 0
  if (r < 1 || r > 64 || !std::isfinite(s)) return QLORA_EINVAL;
  const int64_t k = w.k, n = w.n;
  if (!dims_ok(m, k, n)) return QLORA_ESHAPE;
  if (!src_aligned(w) || !al16(A) || !al16(B) || !al16(dY) || !al16(X) || !al4(U) || !al16(dX) ||
      !al2(dA) || !al2(dB))
    return QLORA_ESHAPE;
  const size_t need = linear_ws(m, k, n, r, mode);
  if (int e = check_ws(ws, ws_bytes, need)) return e;
  hipStream_t st = (hipStream_t)stream;
  if (m == 0) {  // empty batch: zero weight gradients
    PrepJobs J;
    J.zero(r, k, dA, k, 1);
    J.zero(n, r, dB, r, 1);
    QL_TRY(launch_prep(J, st), "linear_bwd: zero grads");
    return QLORA_OK;
  }
  Carver c(ws);
  LinearBwdWs t;
  plan_linear_bwd(c, m, k, n, r, mode, &t);
  const int KE = (int)ceil16(2 * r);
  const int chunks = colreduce_chunks((int)m);

  {  // lt = B^T ; bext = [A^T | A^T | 0]
    PrepJobs J;
    J.copy(B, 1, r, r, n, t.lt, n, 1);
    J.copy(A, 1, k, k, r, t.bext, KE, 1);
    J.copy(A, 1, k, k, r, t.bext + r, KE, 1);
    J.zero(k, KE - 2 * r, t.bext + 2 * r, KE, 1);
    QL_TRY(launch_prep(J, st), "linear_bwd: LoRA layouts");
  }
  // T = dY B
  QL_TRY(launch_rowdot(dY, n, t.lt, n, (int)m, (int)n, (int)r, s, t.t, nullptr, (int)r, r, t.text,
                       KE, KE, t.rpart, st),
         "linear_bwd: T = dY B");
  // dX = dY W + s T A
  if (dX) {
    GemmArgs g = gemm_args();
    g.A = dY; g.lda = n;
    if (staged_like(mode)) {
      if (mode == MODE_BF16)
        QL_TRY(launch_w16_transpose(w.w16, n, k, t.wt, n, 0, st), "linear_bwd: W^T");
      else
        QL_TRY(launch_nf4_dequant_transpose(w.codes, w.amax, n, k, t.wt, n, 0, st),
               "linear_bwd: dequant W^T");
      g.bsrc = BSRC_BF16; g.B = t.wt; g.ldb = n;
    } else {
      g.bsrc = BSRC_NF4_T; g.codes0 = w.codes;
      QL_TRY(fused_absmax(w, t.amx, st, &g.absmax0), "linear_bwd: absmax");
    }
    g.Ae = t.text; g.ldae = KE; g.Be = t.bext; g.ldbe = KE;
    g.M = (int)m; g.N = (int)k; g.K = (int)n; g.KE = KE;
    g.epi = EPI_STORE; g.C = dX; g.ldc = k;
    use_splitk(g, t.kpart);
    QL_TRY(run_gemm(g, r, st), "linear_bwd: dX GEMM");
  }
  // dB = s dY^T U and dA = s T^T X: two jobs of one launch per stage, their
  // partial sets side by side
  {
    ColJobs cj{};
    ColFinishJobs fj{};
    cj.G[0] = dY; cj.ldg[0] = n; cj.C[0] = (int)n; cj.V[0] = U; cj.part[0] = t.part;
    cj.G[1] = X; cj.ldg[1] = k; cj.C[1] = (int)k; cj.V[1] = t.t;
    cj.part[1] = t.part + (int64_t)chunks * n * r;
    fj.part[0] = cj.part[0]; fj.C[0] = (int)n; fj.R[0] = (int)r; fj.j0[0] = 0; fj.out[0] = dB;
    fj.ocs[0] = r; fj.ojs[0] = 1;
    fj.part[1] = cj.part[1]; fj.C[1] = (int)k; fj.R[1] = (int)r; fj.j0[1] = 0; fj.out[1] = dA;
    fj.ocs[1] = 1; fj.ojs[1] = k;
    QL_TRY(launch_colreduce_jobs(cj, 2, nullptr, nullptr, 0, (int)m, r, (int)r, st),
           "linear_bwd: dB, dA partials");
    QL_TRY(launch_colreduce_finish_jobs(fj, 2, chunks, (int)r, s, st), "linear_bwd: dB, dA");
  }
  return QLORA_OK;
}

int qlora_linear_fwd(const uint16_t* X, int64_t m, qlora_nf4 w, const uint16_t* A,
                     const uint16_t* B, int64_t r, float s, uint16_t* Y, float* U_save, int mode,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!valid_mode(mode)) return QLORA_EINVAL;
  return linear_fwd_impl(X, m, src_nf4(w), A, B, r, s, Y, U_save, resolve_mode(mode, m), ws, ws_bytes,
                         stream);
}

size_t qlora_linear_fwd_noalloc_max_bytes(void) { return kScratchBytes; }


int qlora_linear_fwd_noalloc(const uint16_t* X, int64_t m, qlora_nf4 w, const uint16_t* A,
                             const uint16_t* B, int64_t r, float s, uint16_t* Y, float* U_save,
                             int mode, void* stream) {
  if (!valid_mode(mode)) return QLORA_EINVAL;
  const int md = resolve_mode(mode, m);
  const WSrc src = src_nf4(w);
  if (int e = linear_fwd_check(X, m, src, A, B, r, s, Y, U_save, md)) return e;
  const size_t need = linear_fwd_ws(m, w.k, w.n, r, md);
  if (need > kScratchBytes) {
    g_last_error = "linear_fwd_noalloc: this call needs " + std::to_string(need) +
                   " bytes of scratch, more than the " + std::to_string(kScratchBytes) +
                   " the library holds per device (use qlora_linear_fwd with a workspace)";
    return QLORA_EWORKSPACE;
  }
  if (m == 0) return QLORA_OK;
  void* ws = nullptr;
  QL_TRY(scratch_device_ptr(&ws), "linear_fwd_noalloc: scratch address");
  return linear_fwd_impl(X, m, src, A, B, r, s, Y, U_save, md, ws, kScratchBytes, stream, false);
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* U, int64_t m, qlora_nf4 w,
                     const uint16_t* A, const uint16_t* B, int64_t r, float s, uint16_t* dX,
                     uint16_t* dA, uint16_t* dB, int mode, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!valid_mode(mode)) return QLORA_EINVAL;
  return linear_bwd_impl(dY, X, U, m, src_nf4(w), A, B, r, s, dX, dA, dB, resolve_mode(mode, m), ws,
                         ws_bytes, stream);
}

int qlora_linear16_fwd(const uint16_t* X, int64_t m, const uint16_t* W, int64_t n, int64_t k,
                       const uint16_t* A, const uint16_t* B, int64_t r, float s, uint16_t* Y,
                       float* U_save, void* ws, size_t ws_bytes, void* stream) {
  return linear_fwd_impl(X, m, src_w16(W, n, k), A, B, r, s, Y, U_save, MODE_BF16, ws, ws_bytes,
                         stream);
}

int qlora_linear16_bwd(const uint16_t* dY, const uint16_t* X, const float* U, int64_t m,
                       const uint16_t* W, int64_t n, int64_t k, const uint16_t* A,
                       const uint16_t* B, int64_t r, float s, uint16_t* dX, uint16_t* dA,
                       uint16_t* dB, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(dY, X, U, m, src_w16(W, n, k), A, B, r, s, dX, dA, dB, MODE_BF16, ws,
                         ws_bytes, stream);
}

// --------------------------------------------------------------- gated MLP --
// MLP weights with their base-weight sources (NF4 or bf16)
struct MlpSrc {
  WSrc gate, up, down;
  const uint16_t *a_gate, *b_gate, *a_up, *b_up, *a_down, *b_down;
  int64_t d, h, r;
  float s;
  int act;
};

static MlpSrc mlp_src(const qlora_mlp_weights* w) {
  MlpSrc m;
  m.gate = src_nf4(w->gate); m.up = src_nf4(w->up); m.down = src_nf4(w->down);
  m.a_gate = w->a_gate; m.b_gate = w->b_gate; m.a_up = w->a_up; m.b_up = w->b_up;
  m.a_down = w->a_down; m.b_down = w->b_down;
  m.d = w->d; m.h = w->h; m.r = w->r; m.s = w->s; m.act = w->act;
  return m;
}

static MlpSrc mlp_src16(const qlora_mlp16_weights* w) {
  MlpSrc m;
  m.gate = src_w16(w->gate, w->h, w->d); m.up = src_w16(w->up, w->h, w->d);
  m.down = src_w16(w->down, w->d, w->h);
  m.a_gate = w->a_gate; m.b_gate = w->b_gate; m.a_up = w->a_up; m.b_up = w->b_up;
  m.a_down = w->a_down; m.b_down = w->b_down;
  m.d = w->d; m.h = w->h; m.r = w->r; m.s = w->s; m.act = w->act;
  return m;
}

static int check_mlp(const MlpSrc& w, int mode) {
  if (bad_src(w.gate, mode) || bad_src(w.up, mode) || bad_src(w.down, mode)) return QLORA_EINVAL;
  if (!w.a_gate || !w.b_gate || !w.a_up || !w.b_up || !w.a_down || !w.b_down) return QLORA_EINVAL;
  if (w.r < 1 || w.r > 64 || !std::isfinite(w.s)) return QLORA_EINVAL;
  if (w.act != QLORA_ACT_SWIGLU && w.act != QLORA_ACT_GEGLU_TANH) return QLORA_EINVAL;
  const int64_t d = w.d, h = w.h;
  if (!dims_ok(0, d, h)) return QLORA_ESHAPE;
  if (w.gate.n != h || w.gate.k != d || w.up.n != h || w.up.k != d || w.down.n != d || w.down.k != h)
    return QLORA_ESHAPE;
  if (!src_aligned(w.gate) || !src_aligned(w.up) || !src_aligned(w.down)) return QLORA_ESHAPE;
  if (!al16(w.a_gate) || !al16(w.b_gate) || !al16(w.a_up) || !al16(w.b_up) || !al16(w.a_down) ||
      !al16(w.b_down))
    return QLORA_ESHAPE;
  return QLORA_OK;
}

static size_t mlp_ws(int64_t m, int64_t d, int64_t h, int64_t r, int mode) {
  Carver a(nullptr), b(nullptr);
  return std::max(plan_mlp_fwd(a, m, d, h, r, mode, nullptr), plan_mlp_bwd(b, m, d, h, r, mode, nullptr));
}

size_t qlora_mlp_workspace_bytes(int64_t m, int64_t d, int64_t h, int64_t r, int mode) {
  if (!dims_ok(m, d, h) || r < 1 || r > 64 || !valid_mode(mode)) return 0;
  return mlp_ws(m, d, h, r, resolve_mode(mode, m));
}

size_t qlora_mlp16_workspace_bytes(int64_t m, int64_t d, int64_t h, int64_t r) {
  if (!dims_ok(m, d, h) || r < 1 || r > 64) return 0;
  return mlp_ws(m, d, h, r, MODE_BF16);
}

static int mlp_fwd_impl(const uint16_t* X, int64_t m, const MlpSrc* w, uint16_t* Y,
                        uint16_t* g_save, uint16_t* u_save, float* Ug, float* Uu, float* Ud, int mode,
                        void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_mlp(*w, mode)) return e;
  if (m > 0 && (!X || !Y || !g_save || !u_save || !Ug || !Uu || !Ud)) return QLORA_EINVAL;
  const int64_t d = w->d, h = w->h, r = w->r;
  if (m < 0 || m >= ((int64_t)1 << 30)) return QLORA_ESHAPE;
  if (!al16(X) || !al16(Y) || !al16(g_save) || !al16(u_save) || !al4(Ug) || !al4(Uu) || !al4(Ud))
    return QLORA_ESHAPE;
  const size_t need = mlp_ws(m, d, h, r, mode);
  if (int e = check_ws(ws, ws_bytes, need)) return e;
  if (m == 0) return QLORA_OK;
  hipStream_t st = (hipStream_t)stream;
  Carver c(ws);
  MlpFwdWs t;
  plan_mlp_fwd(c, m, d, h, r, mode, &t);
  const int KEgu = (int)mlp_ke_gu(r), KEd = (int)ceil16(2 * r);
  const bool wide = mlp_wide(r);
  const int E = (int)ceil16(2 * r);   // wide: one projection's segment
  const float s = w->s;

  // LoRA operand layouts (launched below: on the helper stream when staged,
  // ahead of the row product there, so the caller's stream starts with the
  // dequant; every reader of these layouts waits for the helper stream)
  PrepJobs fwd_jobs;
  {  // Lgu = [Ag; Au]; Bext_gu rows interleaved by 32 (gate: [Bg 0 Bg 0 0..],
     // up: [0 Bu 0 Bu 0..]; wide: gate [Bg Bg 0.. | 0..], up [0.. | Bu Bu 0..]);
     // Bext_d = [Bd | Bd | 0]
    PrepJobs J;
    J.copy(w->a_gate, d, 1, r, d, t.lgu, d, 1);
    J.copy(w->a_up, d, 1, r, d, t.lgu + r * d, d, 1);
    if (!wide) {
      J.copy(w->b_gate, r, 1, h, r, t.bextgu, KEgu, 1, 1);
      J.zero(h, r, t.bextgu + r, KEgu, 1, 1);
      J.copy(w->b_gate, r, 1, h, r, t.bextgu + 2 * r, KEgu, 1, 1);
      J.zero(h, KEgu - 3 * r, t.bextgu + 3 * r, KEgu, 1, 1);
      J.zero(h, r, t.bextgu, KEgu, 1, 2);
      J.copy(w->b_up, r, 1, h, r, t.bextgu + r, KEgu, 1, 2);
      J.zero(h, r, t.bextgu + 2 * r, KEgu, 1, 2);
      J.copy(w->b_up, r, 1, h, r, t.bextgu + 3 * r, KEgu, 1, 2);
      J.zero(h, KEgu - 4 * r, t.bextgu + 4 * r, KEgu, 1, 2);
    } else {
      J.copy(w->b_gate, r, 1, h, r, t.bextgu, KEgu, 1, 1);
      J.copy(w->b_gate, r, 1, h, r, t.bextgu + r, KEgu, 1, 1);
      J.zero(h, KEgu - 2 * r, t.bextgu + 2 * r, KEgu, 1, 1);
      J.zero(h, E, t.bextgu, KEgu, 1, 2);
      J.copy(w->b_up, r, 1, h, r, t.bextgu + E, KEgu, 1, 2);
      J.copy(w->b_up, r, 1, h, r, t.bextgu + E + r, KEgu, 1, 2);
      J.zero(h, E - 2 * r, t.bextgu + E + 2 * r, KEgu, 1, 2);
    }
    J.copy(w->b_down, r, 1, d, r, t.bextd, KEd, 1);
    J.copy(w->b_down, r, 1, d, r, t.bextd + r, KEd, 1);
    J.zero(d, KEd - 2 * r, t.bextd + 2 * r, KEd, 1);
    fwd_jobs = J;
  }
  // staged: the caller's stream writes the gate/up weight that the first GEMM
  // needs, while the helper stream does the row product [Ug | Uu] and then the
  // down weight; each GEMM waits for exactly what it reads
  const bool staged = staged_like(mode);
  const bool w16 = mode == MODE_BF16;
  Side side(st);
  // [Ug | Uu] = X [Ag; Au]^T  (one read of X for both projections; two when
  // 2r is wider than one row product)
  auto row_u = [&](hipStream_t q) {
    if (!wide)
      return launch_rowdot(X, d, t.lgu, d, (int)m, (int)d, (int)(2 * r), s, Ug, Uu, (int)r, r,
                           t.uextgu, KEgu, KEgu, t.rpart, q);
    // Ug and Uu as two jobs of one launch, each with its own partials
    RowJobs in{};
    RowFinishJobs out{};
    float* uo[2] = {Ug, Uu};
    for (int q2 = 0; q2 < 2; ++q2) {
      in.G[q2] = X; in.ldg[q2] = d; in.L[q2] = t.lgu + q2 * r * d; in.ldl[q2] = d; in.K[q2] = (int)d;
      in.part[q2] = t.rpart + (int64_t)q2 * 16 * m * r;
      out.Uf[q2] = uo[q2]; out.Uf2[q2] = nullptr; out.split[q2] = (int)r; out.ldu[q2] = r;
      out.Ue[q2] = t.uextgu + q2 * E; out.ldue[q2] = KEgu; out.KE[q2] = (int)E;
    }
    return launch_rowdot_jobs(in, out, 2, (int)m, (int)r, s, q);
  };
  if (staged) {
    QL_TRY(side.open(), "mlp_fwd: helper stream");
    QL_TRY(side.fork(0), "mlp_fwd: fork");
    hipStream_t ss = side.stream();
    QL_TRY(launch_prep(fwd_jobs, ss), "mlp_fwd: LoRA layouts");
    QL_TRY(row_u(ss), "mlp_fwd: Ug, Uu");
    QL_TRY(side.mark(1), "mlp_fwd: mark");
    if (w16) {   // 16-bit base: interleave copy of gate/up; down is used as it is
      QL_TRY(launch_w16_rows(w->gate.w16, h, d, t.wgu, d, 1, st), "mlp_fwd: gate/up copy");
      QL_TRY(launch_w16_rows(w->up.w16, h, d, t.wgu, d, 2, st), "mlp_fwd: gate/up copy");
    } else {
      QL_TRY(launch_nf4_dequant_rows(w->gate.codes, w->gate.amax, h, d, t.wgu, d, 1, st), "mlp_fwd: dequant");
      QL_TRY(launch_nf4_dequant_rows(w->up.codes, w->up.amax, h, d, t.wgu, d, 2, st), "mlp_fwd: dequant");
      QL_TRY(launch_nf4_dequant_rows(w->down.codes, w->down.amax, d, h, t.wd, h, 0, ss), "mlp_fwd: dequant");
    }
    QL_TRY(side.mark(2), "mlp_fwd: mark");
  } else {
    QL_TRY(launch_prep(fwd_jobs, st), "mlp_fwd: LoRA layouts");
    QL_TRY(row_u(st), "mlp_fwd: Ug, Uu");
  }
  // gate || up GEMM with the activation epilogue
  GemmArgs g = gemm_args();
  g.A = X; g.lda = d;
  if (staged) { g.bsrc = BSRC_BF16; g.B = t.wgu; g.ldb = d; }
  else {
    g.bsrc = BSRC_NF4_PAIR;
    g.codes0 = w->gate.codes; g.codes1 = w->up.codes;
    QL_TRY(fused_absmax(w->gate, t.amx, st, &g.absmax0), "mlp_fwd: absmax");
    QL_TRY(fused_absmax(w->up, t.amx + h * (d / 64), st, &g.absmax1), "mlp_fwd: absmax");
  }
  g.Ae = t.uextgu; g.ldae = KEgu; g.Be = t.bextgu; g.ldbe = KEgu;
  g.M = (int)m; g.N = (int)(2 * h); g.K = (int)d; g.KE = KEgu;
  g.epi = EPI_GATEUP; g.g_out = g_save; g.u_out = u_save; g.h_out = t.H; g.hdim = h; g.act = w->act;
  // Ud = H Ad^T ; Y = H Wd^T + s Ud Bd^T
  const bool rp = rp_epilogue(r, m);
  if (rp) { g.rp_l = w->a_down; g.rp_ldl = h; g.rp_r = (int)r; g.rp_part = t.rpart; }
  if (staged) QL_TRY(side.wait(1), "mlp_fwd: wait");
  QL_TRY(run_gemm(g, r, st), "mlp_fwd: gate/up GEMM");
  if (rp)
    QL_TRY(launch_rowdot_finish(t.rpart, gemm_rowprod_splits((int)(2 * h)), (int)m, (int)r, s, Ud,
                                nullptr, (int)r, r, t.uextd, KEd, KEd, st),
           "mlp_fwd: Ud");
  else
    QL_TRY(launch_rowdot(t.H, h, w->a_down, h, (int)m, (int)h, (int)r, s, Ud, nullptr, (int)r, r,
                         t.uextd, KEd, KEd, t.rpart, st),
           "mlp_fwd: Ud");
  GemmArgs g2 = gemm_args();
  g2.A = t.H; g2.lda = h;
  if (w16) { g2.bsrc = BSRC_BF16; g2.B = w->down.w16; g2.ldb = h; }
  else if (staged) { g2.bsrc = BSRC_BF16; g2.B = t.wd; g2.ldb = h; }
  else {
    g2.bsrc = BSRC_NF4; g2.codes0 = w->down.codes;
    QL_TRY(fused_absmax(w->down, t.amx + 2 * h * (d / 64), st, &g2.absmax0), "mlp_fwd: absmax");
  }
  g2.Ae = t.uextd; g2.ldae = KEd; g2.Be = t.bextd; g2.ldbe = KEd;
  g2.M = (int)m; g2.N = (int)d; g2.K = (int)h; g2.KE = KEd;
  g2.epi = EPI_STORE; g2.C = Y; g2.ldc = d;
  use_splitk(g2, t.kpart);
  if (staged) QL_TRY(side.wait(2), "mlp_fwd: join");
  QL_TRY(run_gemm(g2, r, st), "mlp_fwd: down GEMM");
  return QLORA_OK;
}

static int mlp_bwd_impl(const uint16_t* dY, const uint16_t* X, const uint16_t* g_save,
                        const uint16_t* u_save, const float* Ug, const float* Uu, const float* Ud,
                        int64_t m, const MlpSrc* w, uint16_t* dX,
                        const qlora_mlp_grads* gr, int mode, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_mlp(*w, mode)) return e;
  if (!gr) return QLORA_EINVAL;
  if (m > 0 && (!dY || !X || !g_save || !u_save || !Ug || !Uu || !Ud)) return QLORA_EINVAL;
  if (!gr->a_gate || !gr->b_gate || !gr->a_up || !gr->b_up || !gr->a_down || !gr->b_down)
    return QLORA_EINVAL;
  const int64_t d = w->d, h = w->h, r = w->r;
  if (m < 0 || m >= ((int64_t)1 << 30)) return QLORA_ESHAPE;
  if (!al16(dY) || !al16(X) || !al16(g_save) || !al16(u_save) || !al4(Ug) || !al4(Uu) ||
      !al4(Ud) || !al16(dX) || !al2(gr->a_gate) || !al2(gr->b_gate) || !al2(gr->a_up) ||
      !al2(gr->b_up) || !al2(gr->a_down) || !al2(gr->b_down))
    return QLORA_ESHAPE;
  const size_t need = mlp_ws(m, d, h, r, mode);
  if (int e = check_ws(ws, ws_bytes, need)) return e;
  hipStream_t st = (hipStream_t)stream;
  if (m == 0) {
    PrepJobs J;
    J.zero(r, d, gr->a_gate, d, 1);
    J.zero(r, d, gr->a_up, d, 1);
    J.zero(r, h, gr->a_down, h, 1);
    J.zero(h, r, gr->b_gate, r, 1);
    J.zero(h, r, gr->b_up, r, 1);
    J.zero(d, r, gr->b_down, r, 1);
    QL_TRY(launch_prep(J, st), "mlp_bwd: zero grads");
    return QLORA_OK;
  }
  Carver c(ws);
  MlpBwdWs t;
  plan_mlp_bwd(c, m, d, h, r, mode, &t);
  const int KEgu = (int)mlp_ke_gu(r), KEd = (int)ceil16(2 * r);
  const bool wide = mlp_wide(r);
  const int E = (int)ceil16(2 * r);   // wide: one projection's segment
  const int chunks = colreduce_chunks((int)m);
  const float s = w->s;

  // LoRA operand layouts (launched below on the caller's stream, before the
  // helper stream forks: everything after reads them)
  PrepJobs bwd_jobs;
  {  // ltd = Bd^T; bextdh = [Ad^T | Ad^T | 0]; ltgu = blockdiag(Bg^T, Bu^T);
     // bextdx = [Ag^T | Au^T | Ag^T | Au^T | 0] (wide: [Ag^T Ag^T 0.. | Au^T Au^T 0..])
    PrepJobs J;
    J.copy(w->b_down, 1, r, r, d, t.ltd, d, 1);
    J.copy(w->a_down, 1, h, h, r, t.bextdh, KEd, 1);
    J.copy(w->a_down, 1, h, h, r, t.bextdh + r, KEd, 1);
    J.zero(h, KEd - 2 * r, t.bextdh + 2 * r, KEd, 1);
    J.copy(w->b_gate, 1, r, r, h, t.ltgu, 2 * h, 1);
    J.zero(r, h, t.ltgu + h, 2 * h, 1);
    J.zero(r, h, t.ltgu + r * 2 * h, 2 * h, 1);
    J.copy(w->b_up, 1, r, r, h, t.ltgu + r * 2 * h + h, 2 * h, 1);
    if (!wide) {
      J.copy(w->a_gate, 1, d, d, r, t.bextdx, KEgu, 1);
      J.copy(w->a_up, 1, d, d, r, t.bextdx + r, KEgu, 1);
      J.copy(w->a_gate, 1, d, d, r, t.bextdx + 2 * r, KEgu, 1);
      J.copy(w->a_up, 1, d, d, r, t.bextdx + 3 * r, KEgu, 1);
      J.zero(d, KEgu - 4 * r, t.bextdx + 4 * r, KEgu, 1);
    } else {
      J.copy(w->a_gate, 1, d, d, r, t.bextdx, KEgu, 1);
      J.copy(w->a_gate, 1, d, d, r, t.bextdx + r, KEgu, 1);
      J.zero(d, E - 2 * r, t.bextdx + 2 * r, KEgu, 1);
      J.copy(w->a_up, 1, d, d, r, t.bextdx + E, KEgu, 1);
      J.copy(w->a_up, 1, d, d, r, t.bextdx + E + r, KEgu, 1);
      J.zero(d, E - 2 * r, t.bextdx + E + 2 * r, KEgu, 1);
    }
    bwd_jobs = J;
  }
  // The column reductions (dB, dA) and the transposed dequant of the gate/up
  // weights run on the helper stream, overlapping the row products and the two
  // GEMMs on the caller's stream; each waits for exactly the tensors it reads.
  // All column reductions share t.part, so they stay in order on one stream.
  const bool staged = staged_like(mode);
  const bool w16 = mode == MODE_BF16;
  Side side(st);
  QL_TRY(side.open(), "mlp_bwd: helper stream");
  hipStream_t ss = side.stream();
  QL_TRY(launch_prep(bwd_jobs, st), "mlp_bwd: LoRA layouts");
  QL_TRY(side.fork(0), "mlp_bwd: fork");
  // Td = dY Bd: on the helper stream beside the caller's W_d^T when staged
  auto row_td = [&](hipStream_t q) {
    return launch_rowdot(dY, d, t.ltd, d, (int)m, (int)d, (int)r, s, t.td, nullptr, (int)r, r,
                         t.textd, KEd, KEd, t.rpart, q);
  };
  if (staged) {
    QL_TRY(row_td(ss), "mlp_bwd: Td");
    QL_TRY(side.mark(2), "mlp_bwd: mark");
  }
  if (w16) {
    QL_TRY(launch_w16_transpose(w->gate.w16, h, d, t.wgut, 2 * h, 0, ss), "mlp_bwd: Wg^T");
    QL_TRY(launch_w16_transpose(w->up.w16, h, d, t.wgut, 2 * h, h, ss), "mlp_bwd: Wu^T");
  } else if (staged) {
    QL_TRY(launch_nf4_dequant_transpose(w->gate.codes, w->gate.amax, h, d, t.wgut, 2 * h, 0, ss),
           "mlp_bwd: dequant Wg^T");
    QL_TRY(launch_nf4_dequant_transpose(w->up.codes, w->up.amax, h, d, t.wgut, 2 * h, h, ss),
           "mlp_bwd: dequant Wu^T");
  }
  QL_TRY(side.mark(1), "mlp_bwd: mark");
  // dBd = s dY^T Ud (inputs only)
  QL_TRY(launch_colreduce(dY, nullptr, nullptr, 0, d, (int)m, (int)d, Ud, r, (int)r, t.part, ss),
         "mlp_bwd: dBd partials");
  QL_TRY(launch_colreduce_finish(t.part, chunks, (int)d, (int)r, 0, (int)r, s, gr->b_down, r, 1, ss),
         "mlp_bwd: dBd");

  // down projection: Td = dY Bd
  if (w16)
    QL_TRY(launch_w16_transpose(w->down.w16, d, h, t.wdt, d, 0, st), "mlp_bwd: Wd^T");
  else if (staged)
    QL_TRY(launch_nf4_dequant_transpose(w->down.codes, w->down.amax, d, h, t.wdt, d, 0, st),
           "mlp_bwd: dequant Wd^T");
  if (staged) {
    QL_TRY(side.wait(2), "mlp_bwd: wait");
  } else {
    QL_TRY(row_td(st), "mlp_bwd: Td");
    QL_TRY(side.fork(2), "mlp_bwd: fork");
  }
  // dAd = s Td^T H, H recomputed from g, u (helper stream, beside the dH GEMM)
  QL_TRY(launch_colreduce(nullptr, g_save, u_save, w->act, h, (int)m, (int)h, t.td, r, (int)r,
                          t.part, ss),
         "mlp_bwd: dAd partials");
  QL_TRY(launch_colreduce_finish(t.part, chunks, (int)h, (int)r, 0, (int)r, s, gr->a_down, 1, h, ss),
         "mlp_bwd: dAd");
  // dH = dY Wd + s Td Ad, with dg, du in the epilogue
  GemmArgs g = gemm_args();
  g.A = dY; g.lda = d;
  if (staged) { g.bsrc = BSRC_BF16; g.B = t.wdt; g.ldb = d; }
  else {
    g.bsrc = BSRC_NF4_T; g.codes0 = w->down.codes;
    QL_TRY(fused_absmax(w->down, t.amx + 2 * h * (d / 64), st, &g.absmax0), "mlp_bwd: absmax");
  }
  g.Ae = t.textd; g.ldae = KEd; g.Be = t.bextdh; g.ldbe = KEd;
  g.M = (int)m; g.N = (int)h; g.K = (int)d; g.KE = KEd;
  g.epi = EPI_ACT_BWD; g.g_in = g_save; g.u_in = u_save; g.dgu = t.dgu; g.hdim = h; g.act = w->act;
  // [Tg | Tu] = [dg | du] blockdiag(Bg, Bu): in the epilogue, or below
  const bool rp = rp_epilogue(r, m);
  if (rp) {
    g.rp_l = t.ltgu; g.rp_l2 = t.ltgu + r * 2 * h + h; g.rp_ldl = 2 * h;
    g.rp_r = (int)r; g.rp_part = t.rpart;
  }
  QL_TRY(run_gemm(g, r, st), "mlp_bwd: dH GEMM");
  QL_TRY(side.fork(3), "mlp_bwd: fork");
  // dBg = s dg^T Ug ; dBu = s du^T Uu (helper stream). Up to kMergedDbTokens
  // tokens the two run as one launch per stage (partial sets side by side):
  // there the launches, not the bytes, decide when the helper is done, and
  // it is on the step's tail. Above, one after the other, which shares the
  // CUs of the dX GEMM beside it more evenly (measured: merged +2.1% at
  // 1024 tokens, -0.3% at 8192).
  {
    const uint16_t* src[2] = {t.dgu, t.dgu + h};
    const float* uu[2] = {Ug, Uu};
    uint16_t* out[2] = {gr->b_gate, gr->b_up};
    const bool merged = m <= kMergedDbTokens;
    ColJobs cj{};
    ColFinishJobs fj{};
    for (int q = 0; q < 2; ++q) {
      float* part = t.part + (merged ? (int64_t)q * chunks * h * r : 0);
      cj.G[q] = src[q]; cj.ldg[q] = 2 * h; cj.C[q] = (int)h; cj.V[q] = uu[q]; cj.part[q] = part;
      fj.part[q] = part; fj.C[q] = (int)h; fj.R[q] = (int)r; fj.j0[q] = 0; fj.out[q] = out[q];
      fj.ocs[q] = r; fj.ojs[q] = 1;
    }
    if (merged) {
      QL_TRY(launch_colreduce_jobs(cj, 2, nullptr, nullptr, 0, (int)m, r, (int)r, ss),
             "mlp_bwd: dBg, dBu partials");
      QL_TRY(launch_colreduce_finish_jobs(fj, 2, chunks, (int)r, s, ss), "mlp_bwd: dBg, dBu");
    } else {
      for (int q = 0; q < 2; ++q) {
        QL_TRY(launch_colreduce(src[q], nullptr, nullptr, 0, 2 * h, (int)m, (int)h, uu[q], r, (int)r,
                                t.part, ss),
               "mlp_bwd: dB partials");
        QL_TRY(launch_colreduce_finish(t.part, chunks, (int)h, (int)r, 0, (int)r, s, out[q], r, 1, ss),
               "mlp_bwd: dB");
      }
    }
  }
  if (rp)
    QL_TRY(launch_rowdot_finish(t.rpart, gemm_rowprod_splits((int)h), (int)m, (int)(2 * r), s,
                                t.tgu, nullptr, (int)(2 * r), 2 * r, t.textgu, KEgu, KEgu, st),
           "mlp_bwd: Tg, Tu");
  else if (!wide)
    QL_TRY(launch_rowdot(t.dgu, 2 * h, t.ltgu, 2 * h, (int)m, (int)(2 * h), (int)(2 * r), s,
                         t.tgu, nullptr, (int)(2 * r), 2 * r, t.textgu, KEgu, KEgu, t.rpart, st),
           "mlp_bwd: Tg, Tu");
  else {   // Tg = dg Bg, Tu = du Bu: one row product each (two jobs of one launch), own K-extension segment
    RowJobs in{};
    RowFinishJobs out{};
    for (int q = 0; q < 2; ++q) {
      in.G[q] = t.dgu + q * h; in.ldg[q] = 2 * h; in.L[q] = t.ltgu + q * (r * 2 * h + h);
      in.ldl[q] = 2 * h; in.K[q] = (int)h; in.part[q] = t.rpart + (int64_t)q * 16 * m * r;
      out.Uf[q] = t.tgu + q * r; out.Uf2[q] = nullptr; out.split[q] = (int)r; out.ldu[q] = 2 * r;
      out.Ue[q] = t.textgu + q * E; out.ldue[q] = KEgu; out.KE[q] = (int)E;
    }
    QL_TRY(launch_rowdot_jobs(in, out, 2, (int)m, (int)r, s, st), "mlp_bwd: Tg, Tu");
  }
  QL_TRY(side.fork(4), "mlp_bwd: fork");
  // dAg = s Tg^T X ; dAu = s Tu^T X (helper stream, beside the dX GEMM)
  if (!wide) {
    QL_TRY(launch_colreduce(X, nullptr, nullptr, 0, d, (int)m, (int)d, t.tgu, 2 * r, (int)(2 * r),
                            t.part, ss),
           "mlp_bwd: dAg, dAu partials");
    ColFinishJobs fj{};
    uint16_t* out[2] = {gr->a_gate, gr->a_up};
    for (int q = 0; q < 2; ++q) {
      fj.part[q] = t.part; fj.C[q] = (int)d; fj.R[q] = (int)(2 * r); fj.j0[q] = (int)(q * r);
      fj.out[q] = out[q]; fj.ocs[q] = 1; fj.ojs[q] = d;
    }
    QL_TRY(launch_colreduce_finish_jobs(fj, 2, chunks, (int)r, s, ss), "mlp_bwd: dAg, dAu");
  } else {   // 2r wider than one column reduction: one per projection
    ColJobs cj{};
    ColFinishJobs fj{};
    uint16_t* out[2] = {gr->a_gate, gr->a_up};
    for (int q = 0; q < 2; ++q) {
      float* part = t.part + (int64_t)q * chunks * d * r;
      cj.G[q] = X; cj.ldg[q] = d; cj.C[q] = (int)d; cj.V[q] = t.tgu + q * r; cj.part[q] = part;
      fj.part[q] = part; fj.C[q] = (int)d; fj.R[q] = (int)r; fj.j0[q] = 0; fj.out[q] = out[q];
      fj.ocs[q] = 1; fj.ojs[q] = d;
    }
    QL_TRY(launch_colreduce_jobs(cj, 2, nullptr, nullptr, 0, (int)m, 2 * r, (int)r, ss),
           "mlp_bwd: dAg, dAu partials");
    QL_TRY(launch_colreduce_finish_jobs(fj, 2, chunks, (int)r, s, ss), "mlp_bwd: dAg, dAu");
  }
  // dX = [dg | du] [Wg; Wu] + s [Tg | Tu] [Ag; Au]
  if (dX) {
    GemmArgs g2 = gemm_args();
    g2.A = t.dgu; g2.lda = 2 * h;
    if (staged) { g2.bsrc = BSRC_BF16; g2.B = t.wgut; g2.ldb = 2 * h; }
    else {
      g2.bsrc = BSRC_NF4_T;
      g2.codes0 = w->gate.codes; g2.codes1 = w->up.codes;
      QL_TRY(fused_absmax(w->gate, t.amx, st, &g2.absmax0), "mlp_bwd: absmax");
      QL_TRY(fused_absmax(w->up, t.amx + h * (d / 64), st, &g2.absmax1), "mlp_bwd: absmax");
      g2.ksplit = (int)h;
    }
    g2.Ae = t.textgu; g2.ldae = KEgu; g2.Be = t.bextdx; g2.ldbe = KEgu;
    g2.M = (int)m; g2.N = (int)d; g2.K = (int)(2 * h); g2.KE = KEgu;
    g2.epi = EPI_STORE; g2.C = dX; g2.ldc = d;
    use_splitk(g2, t.kpart);
    QL_TRY(side.wait(1), "mlp_bwd: wait");   // transposed gate/up weights
    QL_TRY(run_gemm(g2, 2 * r, st), "mlp_bwd: dX GEMM");
  }
  QL_TRY(side.join(5), "mlp_bwd: join");
  return QLORA_OK;
}

int qlora_mlp_fwd(const uint16_t* X, int64_t m, const qlora_mlp_weights* w, uint16_t* Y,
                  uint16_t* g_save, uint16_t* u_save, float* Ug, float* Uu, float* Ud, int mode,
                  void* ws, size_t ws_bytes, void* stream) {
  if (!w || !valid_mode(mode)) return QLORA_EINVAL;
  const MlpSrc src = mlp_src(w);
  return mlp_fwd_impl(X, m, &src, Y, g_save, u_save, Ug, Uu, Ud, resolve_mode(mode, m), ws, ws_bytes,
                      stream);
}

int qlora_mlp_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* g_save,
                  const uint16_t* u_save, const float* Ug, const float* Uu, const float* Ud,
                  int64_t m, const qlora_mlp_weights* w, uint16_t* dX,
                  const qlora_mlp_grads* gr, int mode, void* ws, size_t ws_bytes, void* stream) {
  if (!w || !valid_mode(mode)) return QLORA_EINVAL;
  const MlpSrc src = mlp_src(w);
  return mlp_bwd_impl(dY, X, g_save, u_save, Ug, Uu, Ud, m, &src, dX, gr, resolve_mode(mode, m), ws,
                      ws_bytes, stream);
}

int qlora_mlp16_fwd(const uint16_t* X, int64_t m, const qlora_mlp16_weights* w, uint16_t* Y,
                    uint16_t* g_save, uint16_t* u_save, float* Ug, float* Uu, float* Ud,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!w) return QLORA_EINVAL;
  const MlpSrc src = mlp_src16(w);
  return mlp_fwd_impl(X, m, &src, Y, g_save, u_save, Ug, Uu, Ud, MODE_BF16, ws, ws_bytes, stream);
}

int qlora_mlp16_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* g_save,
                    const uint16_t* u_save, const float* Ug, const float* Uu, const float* Ud,
                    int64_t m, const qlora_mlp16_weights* w, uint16_t* dX,
                    const qlora_mlp_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  if (!w) return QLORA_EINVAL;
  const MlpSrc src = mlp_src16(w);
  return mlp_bwd_impl(dY, X, g_save, u_save, Ug, Uu, Ud, m, &src, dX, gr, MODE_BF16, ws, ws_bytes,
                      stream);
}

// ------------------------------------------- q, k, v on one shared input --
// Projection p in {q, k, v} = {0, 1, 2}: Y_p = X W_p^T + s (X A_p^T) B_p^T.
// Forward: one GEMM over the concatenated output width nt = n_q + n_k + n_v
// (B = [W_q; W_k; W_v] in the workspace), the three LoRA terms as one
// K-extension, and an epilogue that writes each column range to its output.
// Backward: dX = sum_p dY_p W_p + s T_p A_p as one GEMM whose K runs over the
// three dY_p (read in place, each with its own pitch).
struct QkvSrc {
  WSrc w[3];
  const uint16_t* a[3];
  const uint16_t* b[3];
  int64_t r;
  float s;
};

static QkvSrc qkv_src(const qlora_qkv_weights* w) {
  QkvSrc q;
  q.w[0] = src_nf4(w->q); q.w[1] = src_nf4(w->k); q.w[2] = src_nf4(w->v);
  q.a[0] = w->a_q; q.a[1] = w->a_k; q.a[2] = w->a_v;
  q.b[0] = w->b_q; q.b[1] = w->b_k; q.b[2] = w->b_v;
  q.r = w->r; q.s = w->s;
  return q;
}

static QkvSrc qkv_src16(const qlora_qkv16_weights* w) {
  QkvSrc q;
  q.w[0] = src_w16(w->q, w->n_q, w->d); q.w[1] = src_w16(w->k, w->n_k, w->d);
  q.w[2] = src_w16(w->v, w->n_v, w->d);
  q.a[0] = w->a_q; q.a[1] = w->a_k; q.a[2] = w->a_v;
  q.b[0] = w->b_q; q.b[1] = w->b_k; q.b[2] = w->b_v;
  q.r = w->r; q.s = w->s;
  return q;
}

static bool qkv_dims_ok(int64_t m, int64_t d, const int64_t n[3]) {
  const int64_t lim = (int64_t)1 << 30;
  if (!dims_ok(m, d, n[0]) || !dims_ok(m, d, n[1]) || !dims_ok(m, d, n[2])) return false;
  return n[0] + n[1] + n[2] < lim;
}

static int check_qkv(const QkvSrc& w, int mode) {
  for (int p = 0; p < 3; ++p)
    if (bad_src(w.w[p], mode) || !w.a[p] || !w.b[p]) return QLORA_EINVAL;
  if (w.r < 1 || w.r > 64 || !std::isfinite(w.s)) return QLORA_EINVAL;
  const int64_t n[3] = {w.w[0].n, w.w[1].n, w.w[2].n};
  const int64_t d = w.w[0].k;
  if (w.w[1].k != d || w.w[2].k != d || !qkv_dims_ok(0, d, n)) return QLORA_ESHAPE;
  for (int p = 0; p < 3; ++p)
    if (!src_aligned(w.w[p]) || !al16(w.a[p]) || !al16(w.b[p])) return QLORA_ESHAPE;
  return QLORA_OK;
}

// a per-token tensor with a row pitch: pitch >= width, 16-byte rows
static bool pitch_ok(const void* p, int64_t ld, int64_t width) {
  return ld >= width && ld % 8 == 0 && ((uintptr_t)p & 15) == 0;
}

// K-extension layout of the forward: with 3r <= 64 one row product forms
// [U_q | U_k | U_v] and the columns are [hi(sU) | lo(sU)] over all three;
// otherwise each projection has its own row product and the columns are
// [hi(sU_q) lo(sU_q) | hi(sU_k) lo(sU_k) | hi(sU_v) lo(sU_v)]. The backward
// always uses the second form (its T_p come from three different dY_p).
struct QkvExt {
  bool one;
  int64_t r;
  int64_t hi(int p) const { return one ? p * r : 2 * r * p; }
  int64_t lo(int p) const { return one ? 3 * r + p * r : 2 * r * p + r; }
};

struct QkvFwdWs {
  uint16_t* lqkv;   // [3r][d]   [A_q; A_k; A_v] (one row product)
  uint16_t* bext;   // [nt][KE]  B_p at its hi and lo columns
  uint16_t* uext;   // [m][KE]
  uint16_t* wcat;   // [nt][d]   [W_q; W_k; W_v] in bf16
  float* rpart;     // row-product split partials
  float* kpart;     // split-K partials of the GEMM
};

static size_t plan_qkv_fwd(Carver& c, int64_t m, int64_t d, int64_t nt, int64_t r, QkvFwdWs* w) {
  const int64_t KE = ceil16(6 * r);
  QkvFwdWs t;
  t.lqkv = c.take<uint16_t>(3 * r * d);
  t.bext = c.take<uint16_t>(nt * KE);
  t.uext = c.take<uint16_t>(m * KE);
  t.wcat = c.take<uint16_t>(nt * d);
  t.rpart = c.take<float>(16 * m * 3 * r);
  t.kpart = c.take<float>(splitk_elems(m, nt, d));
  if (w) *w = t;
  return c.off;
}

struct QkvBwdWs {
  uint16_t* lt;     // [r][nt]   [B_q^T | B_k^T | B_v^T]
  uint16_t* bext;   // [d][KE]   A_p^T at columns 2rp and 2rp + r
  float* t;         // [m][3r]   [T_q | T_k | T_v]
  uint16_t* text;   // [m][KE]
  float* part;      // column-reduction partials
  uint16_t* wt;     // [d][nt]   [W_q^T | W_k^T | W_v^T] in bf16
  float* rpart;     // row-product split partials
  float* kpart;     // split-K partials of the dX GEMM
};

static size_t plan_qkv_bwd(Carver& c, int64_t m, int64_t d, const int64_t n[3], int64_t r,
                           QkvBwdWs* w) {
  const int64_t KE = ceil16(6 * r), nt = n[0] + n[1] + n[2];
  const int64_t chunks = colreduce_chunks((int)std::max<int64_t>(m, 1));
  QkvBwdWs t;
  t.lt = c.take<uint16_t>(r * nt);
  t.bext = c.take<uint16_t>(d * KE);
  t.t = c.take<float>(m * 3 * r);
  t.text = c.take<uint16_t>(m * KE);
  // partials of the column reductions: the three dB_p sets side by side, then
  // the dA sets (one [d][3r] set, or three [d][r] sets side by side)
  t.part = c.take<float>(chunks * std::max(nt * r, 3 * d * r));
  t.wt = c.take<uint16_t>(d * nt);
  t.rpart = c.take<float>(3 * 16 * m * r);   // the three T_p row products' partials
  t.kpart = c.take<float>(splitk_elems(m, d, nt));
  if (w) *w = t;
  return c.off;
}

static size_t qkv_ws(int64_t m, int64_t d, const int64_t n[3], int64_t r) {
  Carver a(nullptr), b(nullptr);
  return std::max(plan_qkv_fwd(a, m, d, n[0] + n[1] + n[2], r, nullptr),
                  plan_qkv_bwd(b, m, d, n, r, nullptr));
}

size_t qlora_qkv_workspace_bytes(int64_t m, int64_t d, int64_t n_q, int64_t n_k, int64_t n_v,
                                 int64_t r) {
  const int64_t n[3] = {n_q, n_k, n_v};
  if (!qkv_dims_ok(m, d, n) || r < 1 || r > 64) return 0;
  return qkv_ws(m, d, n, r);
}

static int qkv_fwd_impl(const uint16_t* X, int64_t m, const QkvSrc& w, uint16_t* const out[3],
                        const int64_t ld[3], float* U, int mode, void* ws, size_t ws_bytes,
                        void* stream) {
  if (int e = check_qkv(w, mode)) return e;
  const int64_t d = w.w[0].k, r = w.r;
  const int64_t n[3] = {w.w[0].n, w.w[1].n, w.w[2].n};
  const int64_t off[3] = {0, n[0], n[0] + n[1]}, nt = n[0] + n[1] + n[2];
  if (m < 0 || m >= ((int64_t)1 << 30)) return QLORA_ESHAPE;
  if (m > 0) {
    if (!X || !U || !out[0] || !out[1] || !out[2]) return QLORA_EINVAL;
    for (int p = 0; p < 3; ++p)
      if (!pitch_ok(out[p], ld[p], n[p])) return QLORA_ESHAPE;
    if (!al16(X) || !al4(U)) return QLORA_ESHAPE;
  }
  if (int e = check_ws(ws, ws_bytes, qkv_ws(m, d, n, r))) return e;
  if (m == 0) return QLORA_OK;
  hipStream_t st = (hipStream_t)stream;
  Carver c(ws);
  QkvFwdWs t;
  plan_qkv_fwd(c, m, d, nt, r, &t);
  const int64_t KE = ceil16(6 * r);
  const QkvExt ex{3 * r <= 64, r};
  const float s = w.s;

  // LoRA operand layouts, one launch: each row block of Bext holds its own
  // projection's B at the hi and lo columns and zeros in the rest of the row
  {
    PrepJobs J;
    for (int p = 0; p < 3; ++p) {
      if (ex.one) J.copy(w.a[p], d, 1, r, d, t.lqkv + p * r * d, d, 1);
      uint16_t* rows = t.bext + off[p] * KE;
      const int64_t h0 = ex.hi(p), l0 = ex.lo(p);   // h0 + r <= l0
      J.copy(w.b[p], r, 1, n[p], r, rows + h0, KE, 1);
      J.copy(w.b[p], r, 1, n[p], r, rows + l0, KE, 1);
      J.zero(n[p], h0, rows, KE, 1);
      J.zero(n[p], l0 - h0 - r, rows + h0 + r, KE, 1);
      J.zero(n[p], KE - l0 - r, rows + l0 + r, KE, 1);
    }
    if (!ex.one) J.zero(m, KE - 6 * r, t.uext + 6 * r, KE, 1);
    QL_TRY(launch_prep(J, st), "qkv_fwd: LoRA layouts");
  }
  // the bf16 copy of [W_q; W_k; W_v] is made on the helper stream while the
  // caller's stream forms the row products
  const bool w16 = mode == MODE_BF16;
  Side side(st);
  QL_TRY(side.open(), "qkv_fwd: helper stream");
  QL_TRY(side.fork(0), "qkv_fwd: fork");
  hipStream_t ss = side.stream();
  for (int p = 0; p < 3; ++p) {
    uint16_t* dst = t.wcat + off[p] * d;
    if (w16)
      QL_TRY(launch_w16_rows(w.w[p].w16, n[p], d, dst, d, 0, ss), "qkv_fwd: weight copy");
    else
      QL_TRY(launch_nf4_dequant_rows(w.w[p].codes, w.w[p].amax, n[p], d, dst, d, 0, ss),
             "qkv_fwd: dequant");
  }
  QL_TRY(side.mark(1), "qkv_fwd: mark");
  if (ex.one) {   // [U_q | U_k | U_v] = X [A_q; A_k; A_v]^T, one read of X
    QL_TRY(launch_rowdot(X, d, t.lqkv, d, (int)m, (int)d, (int)(3 * r), s, U, nullptr,
                         (int)(3 * r), 3 * r, t.uext, KE, (int)KE, t.rpart, st),
           "qkv_fwd: U");
  } else {   // one row product per projection: three jobs of one launch, own partials
    RowJobs in{};
    RowFinishJobs out{};
    for (int p = 0; p < 3; ++p) {
      in.G[p] = X; in.ldg[p] = d; in.L[p] = w.a[p]; in.ldl[p] = d; in.K[p] = (int)d;
      in.part[p] = t.rpart + (int64_t)p * 16 * m * r;
      out.Uf[p] = U + p * r; out.Uf2[p] = nullptr; out.split[p] = (int)r; out.ldu[p] = 3 * r;
      out.Ue[p] = t.uext + ex.hi(p); out.ldue[p] = KE; out.KE[p] = (int)(2 * r);
    }
    QL_TRY(launch_rowdot_jobs(in, out, 3, (int)m, (int)r, s, st), "qkv_fwd: U");
  }
  GemmArgs g = gemm_args();
  g.A = X; g.lda = d;
  g.bsrc = BSRC_BF16; g.B = t.wcat; g.ldb = d;
  g.Ae = t.uext; g.ldae = KE; g.Be = t.bext; g.ldbe = KE;
  g.M = (int)m; g.N = (int)nt; g.K = (int)d; g.KE = (int)KE;
  g.epi = EPI_STORE3;
  g.C = out[0]; g.ldc = ld[0]; g.C1 = out[1]; g.ldc1 = ld[1]; g.C2 = out[2]; g.ldc2 = ld[2];
  g.nc1 = (int)off[1]; g.nc2 = (int)off[2];
  use_splitk(g, t.kpart);
  QL_TRY(side.wait(1), "qkv_fwd: wait");
  QL_TRY(run_gemm(g, r, st), "qkv_fwd: GEMM");
  return QLORA_OK;
}

static int qkv_bwd_impl(const uint16_t* const dy[3], const int64_t lddy[3], const uint16_t* X,
                        const float* U, int64_t m, const QkvSrc& w, uint16_t* dX,
                        const qlora_qkv_grads* gr, int mode, void* ws, size_t ws_bytes,
                        void* stream) {
  if (int e = check_qkv(w, mode)) return e;
  if (!gr || !gr->a_q || !gr->b_q || !gr->a_k || !gr->b_k || !gr->a_v || !gr->b_v)
    return QLORA_EINVAL;
  uint16_t* const ga[3] = {gr->a_q, gr->a_k, gr->a_v};
  uint16_t* const gb[3] = {gr->b_q, gr->b_k, gr->b_v};
  const int64_t d = w.w[0].k, r = w.r;
  const int64_t n[3] = {w.w[0].n, w.w[1].n, w.w[2].n};
  const int64_t off[3] = {0, n[0], n[0] + n[1]}, nt = n[0] + n[1] + n[2];
  if (m < 0 || m >= ((int64_t)1 << 30)) return QLORA_ESHAPE;
  if (m > 0) {
    if (!X || !U || !dy[0] || !dy[1] || !dy[2]) return QLORA_EINVAL;
    for (int p = 0; p < 3; ++p)
      if (!pitch_ok(dy[p], lddy[p], n[p])) return QLORA_ESHAPE;
    if (!al16(X) || !al4(U) || !al16(dX)) return QLORA_ESHAPE;
  }
  for (int p = 0; p < 3; ++p)
    if (!al2(ga[p]) || !al2(gb[p])) return QLORA_ESHAPE;
  if (int e = check_ws(ws, ws_bytes, qkv_ws(m, d, n, r))) return e;
  hipStream_t st = (hipStream_t)stream;
  if (m == 0) {
    PrepJobs J;
    for (int p = 0; p < 3; ++p) {
      J.zero(r, d, ga[p], d, 1);
      J.zero(n[p], r, gb[p], r, 1);
    }
    QL_TRY(launch_prep(J, st), "qkv_bwd: zero grads");
    return QLORA_OK;
  }
  Carver c(ws);
  QkvBwdWs t;
  plan_qkv_bwd(c, m, d, n, r, &t);
  const int64_t KE = ceil16(6 * r);
  const int chunks = colreduce_chunks((int)m);
  const bool one_a = 3 * r <= 64;
  const float s = w.s;

  {  // lt = [B_q^T | B_k^T | B_v^T]; bext rows: A_p^T at columns 2rp and 2rp + r
    PrepJobs J;
    for (int p = 0; p < 3; ++p) {
      J.copy(w.b[p], 1, r, r, n[p], t.lt + off[p], nt, 1);
      J.copy(w.a[p], 1, d, d, r, t.bext + 2 * r * p, KE, 1);
      J.copy(w.a[p], 1, d, d, r, t.bext + 2 * r * p + r, KE, 1);
    }
    J.zero(d, KE - 6 * r, t.bext + 6 * r, KE, 1);
    J.zero(m, KE - 6 * r, t.text + 6 * r, KE, 1);
    QL_TRY(launch_prep(J, st), "qkv_bwd: LoRA layouts");
  }
  // helper stream: the transposed bf16 weights, then dB_p (inputs only), then
  // dA_p once the T_p exist; the caller's stream: T_p, then the dX GEMM
  const bool w16 = mode == MODE_BF16;
  Side side(st);
  QL_TRY(side.open(), "qkv_bwd: helper stream");
  hipStream_t ss = side.stream();
  QL_TRY(side.fork(0), "qkv_bwd: fork");
  if (dX) {
    for (int p = 0; p < 3; ++p) {
      if (w16)
        QL_TRY(launch_w16_transpose(w.w[p].w16, n[p], d, t.wt, nt, off[p], ss), "qkv_bwd: W^T");
      else
        QL_TRY(launch_nf4_dequant_transpose(w.w[p].codes, w.w[p].amax, n[p], d, t.wt, nt, off[p],
                                            ss),
               "qkv_bwd: dequant W^T");
    }
  }
  QL_TRY(side.mark(1), "qkv_bwd: mark");
  {   // dB_p = s dY_p^T U_p: the three in one launch per stage, partial sets side by side
    ColJobs cj{};
    ColFinishJobs fj{};
    int64_t po = 0;
    for (int p = 0; p < 3; ++p) {
      float* part = t.part + po;
      po += (int64_t)chunks * n[p] * r;
      cj.G[p] = dy[p]; cj.ldg[p] = lddy[p]; cj.C[p] = (int)n[p]; cj.V[p] = U + p * r;
      cj.part[p] = part;
      fj.part[p] = part; fj.C[p] = (int)n[p]; fj.R[p] = (int)r; fj.j0[p] = 0; fj.out[p] = gb[p];
      fj.ocs[p] = r; fj.ojs[p] = 1;
    }
    QL_TRY(launch_colreduce_jobs(cj, 3, nullptr, nullptr, 0, (int)m, 3 * r, (int)r, ss),
           "qkv_bwd: dB partials");
    QL_TRY(launch_colreduce_finish_jobs(fj, 3, chunks, (int)r, s, ss), "qkv_bwd: dB");
  }
  {   // T_p = dY_p B_p, and [hi(sT_p) | lo(sT_p)]: three jobs of one launch, own partials
    RowJobs in{};
    RowFinishJobs out{};
    for (int p = 0; p < 3; ++p) {
      in.G[p] = dy[p]; in.ldg[p] = lddy[p]; in.L[p] = t.lt + off[p]; in.ldl[p] = nt;
      in.K[p] = (int)n[p]; in.part[p] = t.rpart + (int64_t)p * 16 * m * r;
      out.Uf[p] = t.t + p * r; out.Uf2[p] = nullptr; out.split[p] = (int)r; out.ldu[p] = 3 * r;
      out.Ue[p] = t.text + 2 * r * p; out.ldue[p] = KE; out.KE[p] = (int)(2 * r);
    }
    QL_TRY(launch_rowdot_jobs(in, out, 3, (int)m, (int)r, s, st), "qkv_bwd: T");
  }
  QL_TRY(side.fork(2), "qkv_bwd: fork");
  if (one_a) {   // dA_p = s T_p^T X, one read of X for all three
    QL_TRY(launch_colreduce(X, nullptr, nullptr, 0, d, (int)m, (int)d, t.t, 3 * r, (int)(3 * r),
                            t.part, ss),
           "qkv_bwd: dA partials");
    ColFinishJobs fj{};
    for (int p = 0; p < 3; ++p) {
      fj.part[p] = t.part; fj.C[p] = (int)d; fj.R[p] = (int)(3 * r); fj.j0[p] = (int)(p * r);
      fj.out[p] = ga[p]; fj.ocs[p] = 1; fj.ojs[p] = d;
    }
    QL_TRY(launch_colreduce_finish_jobs(fj, 3, chunks, (int)r, s, ss), "qkv_bwd: dA");
  } else {   // one reduction per projection, the three in one launch per stage
    ColJobs cj{};
    ColFinishJobs fj{};
    for (int p = 0; p < 3; ++p) {
      float* part = t.part + (int64_t)p * chunks * d * r;
      cj.G[p] = X; cj.ldg[p] = d; cj.C[p] = (int)d; cj.V[p] = t.t + p * r; cj.part[p] = part;
      fj.part[p] = part; fj.C[p] = (int)d; fj.R[p] = (int)r; fj.j0[p] = 0; fj.out[p] = ga[p];
      fj.ocs[p] = 1; fj.ojs[p] = d;
    }
    QL_TRY(launch_colreduce_jobs(cj, 3, nullptr, nullptr, 0, (int)m, 3 * r, (int)r, ss),
           "qkv_bwd: dA partials");
    QL_TRY(launch_colreduce_finish_jobs(fj, 3, chunks, (int)r, s, ss), "qkv_bwd: dA");
  }
  if (dX) {   // dX = [dY_q | dY_k | dY_v] [W_q; W_k; W_v] + s [T_q | T_k | T_v] [A_q; A_k; A_v]
    GemmArgs g = gemm_args();
    g.A = dy[0]; g.lda = lddy[0];
    g.A1 = dy[1]; g.lda1 = lddy[1];
    g.A2 = dy[2]; g.lda2 = lddy[2];
    g.ka1 = (int)off[1]; g.ka2 = (int)off[2];
    g.bsrc = BSRC_BF16; g.B = t.wt; g.ldb = nt;
    g.Ae = t.text; g.ldae = KE; g.Be = t.bext; g.ldbe = KE;
    g.M = (int)m; g.N = (int)d; g.K = (int)nt; g.KE = (int)KE;
    g.epi = EPI_STORE; g.C = dX; g.ldc = d;
    use_splitk(g, t.kpart);
    QL_TRY(side.wait(1), "qkv_bwd: wait");
    QL_TRY(run_gemm(g, 3 * r, st), "qkv_bwd: dX GEMM");
  }
  QL_TRY(side.join(3), "qkv_bwd: join");
  return QLORA_OK;
}

int qlora_qkv_fwd(const uint16_t* X, int64_t m, const qlora_qkv_weights* w, uint16_t* Q,
                  int64_t ld_q, uint16_t* K, int64_t ld_k, uint16_t* V, int64_t ld_v, float* U_save,
                  void* ws, size_t ws_bytes, void* stream) {
  if (!w) return QLORA_EINVAL;
  uint16_t* const out[3] = {Q, K, V};
  const int64_t ld[3] = {ld_q, ld_k, ld_v};
  return qkv_fwd_impl(X, m, qkv_src(w), out, ld, U_save, QLORA_DEQUANT_STAGED, ws, ws_bytes, stream);
}

int qlora_qkv_bwd(const uint16_t* dQ, int64_t ld_dq, const uint16_t* dK, int64_t ld_dk,
                  const uint16_t* dV, int64_t ld_dv, const uint16_t* X, const float* U, int64_t m,
                  const qlora_qkv_weights* w, uint16_t* dX, const qlora_qkv_grads* grads, void* ws,
                  size_t ws_bytes, void* stream) {
  if (!w) return QLORA_EINVAL;
  const uint16_t* const dy[3] = {dQ, dK, dV};
  const int64_t ld[3] = {ld_dq, ld_dk, ld_dv};
  return qkv_bwd_impl(dy, ld, X, U, m, qkv_src(w), dX, grads, QLORA_DEQUANT_STAGED, ws, ws_bytes,
                      stream);
}

int qlora_qkv16_fwd(const uint16_t* X, int64_t m, const qlora_qkv16_weights* w, uint16_t* Q,
                    int64_t ld_q, uint16_t* K, int64_t ld_k, uint16_t* V, int64_t ld_v,
                    float* U_save, void* ws, size_t ws_bytes, void* stream) {
  if (!w) return QLORA_EINVAL;
  uint16_t* const out[3] = {Q, K, V};
  const int64_t ld[3] = {ld_q, ld_k, ld_v};
  return qkv_fwd_impl(X, m, qkv_src16(w), out, ld, U_save, MODE_BF16, ws, ws_bytes, stream);
}

int qlora_qkv16_bwd(const uint16_t* dQ, int64_t ld_dq, const uint16_t* dK, int64_t ld_dk,
                    const uint16_t* dV, int64_t ld_dv, const uint16_t* X, const float* U, int64_t m,
                    const qlora_qkv16_weights* w, uint16_t* dX, const qlora_qkv_grads* grads,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!w) return QLORA_EINVAL;
  const uint16_t* const dy[3] = {dQ, dK, dV};
  const int64_t ld[3] = {ld_dq, ld_dk, ld_dv};
  return qkv_bwd_impl(dy, ld, X, U, m, qkv_src16(w), dX, grads, MODE_BF16, ws, ws_bytes, stream);
}

// ---------------------------------------- RMS layernorm, RoPE, cross entropy --

int qlora_rmsnorm_fwd(const uint16_t* X, int64_t m, int64_t d, const uint16_t* w, float eps,
                      int gemma, uint16_t* Y, float* rstd, void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 33) || d <= 0 || d % 8 || d >= ((int64_t)1 << 30)) return QLORA_ESHAPE;
  if (!w || !std::isfinite(eps) || eps < 0.0f || (gemma != 0 && gemma != 1)) return QLORA_EINVAL;
  if (m == 0) return QLORA_OK;
  if (!X || !Y || !rstd) return QLORA_EINVAL;
  if (!al16(X) || !al16(Y) || !al16(w) || ((uintptr_t)rstd & 3)) return QLORA_ESHAPE;
  QL_TRY(launch_rmsnorm_fwd(X, m, d, w, eps, gemma, Y, rstd, (hipStream_t)stream), "rmsnorm_fwd");
  return QLORA_OK;
}

int qlora_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const float* rstd, int64_t m, int64_t d,
                      const uint16_t* w, int gemma, uint16_t* dX, void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 33) || d <= 0 || d % 8 || d >= ((int64_t)1 << 30)) return QLORA_ESHAPE;
  if (!w || (gemma != 0 && gemma != 1)) return QLORA_EINVAL;
  if (m == 0) return QLORA_OK;
  if (!dY || !X || !rstd || !dX) return QLORA_EINVAL;
  if (!al16(dY) || !al16(X) || !al16(w) || !al16(dX) || ((uintptr_t)rstd & 3)) return QLORA_ESHAPE;
  QL_TRY(launch_rmsnorm_bwd(dY, X, rstd, m, d, w, gemma, dX, (hipStream_t)stream), "rmsnorm_bwd");
  return QLORA_OK;
}

static int rope_impl(const uint16_t* X, int64_t ldx, int64_t m, int64_t heads, int64_t hd,
                     const int64_t* pos, float base, uint16_t* Y, int64_t ldy, int backward,
                     void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 31) || heads < 1 || heads > 4096 || hd < 16 || hd > 256 || hd % 16)
    return QLORA_ESHAPE;
  if (!std::isfinite(base) || base <= 0.0f) return QLORA_EINVAL;
  if (m == 0) return QLORA_OK;
  if (!X || !Y || !pos) return QLORA_EINVAL;
  const int64_t width = heads * hd;
  if (ldx < width || ldy < width || ldx % 8 || ldy % 8 || !al16(X) || !al16(Y)) return QLORA_ESHAPE;
  if (X == Y && ldx != ldy) return QLORA_EINVAL;   // in place only with the same pitch
  if (((uintptr_t)pos & 7)) return QLORA_ESHAPE;
  RopeFreq fr;
  for (int j = 0; j < 128; ++j) fr.inv_freq[j] = j < hd / 2 ? std::pow((double)base, -2.0 * j / (double)hd) : 0.0;
  QL_TRY(launch_rope(X, ldx, Y, ldy, m, (int)heads, (int)hd, pos, fr, backward, (hipStream_t)stream),
         backward ? "rope_bwd" : "rope_fwd");
  return QLORA_OK;
}

int qlora_rope_fwd(const uint16_t* X, int64_t ld_x, int64_t m, int64_t heads, int64_t head_dim,
                   const int64_t* pos, float base, uint16_t* Y, int64_t ld_y, void* stream) {
  return rope_impl(X, ld_x, m, heads, head_dim, pos, base, Y, ld_y, 0, stream);
}

int qlora_rope_bwd(const uint16_t* dY, int64_t ld_dy, int64_t m, int64_t heads, int64_t head_dim,
                   const int64_t* pos, float base, uint16_t* dX, int64_t ld_dx, void* stream) {
  return rope_impl(dY, ld_dy, m, heads, head_dim, pos, base, dX, ld_dx, 1, stream);
}

int qlora_cross_entropy_fwd(const uint16_t* logits, int64_t ld, int64_t m, int64_t V,
                            const int64_t* labels, float* lse, float* ce_rows, float* loss,
                            int32_t* n_valid, void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 31) || V < 1 || V >= ((int64_t)1 << 40) || ld < V || ld % 8)
    return QLORA_ESHAPE;
  if (!loss || !n_valid) return QLORA_EINVAL;
  if (m > 0 && (!logits || !labels || !lse || !ce_rows)) return QLORA_EINVAL;
  if (m > 0 && (!al16(logits) || ((uintptr_t)labels & 7) || ((uintptr_t)lse & 3) ||
                ((uintptr_t)ce_rows & 3)))
    return QLORA_ESHAPE;
  if (((uintptr_t)loss & 3) || ((uintptr_t)n_valid & 3)) return QLORA_ESHAPE;
  QL_TRY(launch_xent_fwd(logits, ld, m, V, labels, lse, ce_rows, loss, n_valid, (hipStream_t)stream),
         "cross_entropy_fwd");
  return QLORA_OK;
}

int qlora_cross_entropy_bwd(const uint16_t* logits, int64_t ld, int64_t m, int64_t V,
                            const int64_t* labels, const float* lse, const float* dloss,
                            const int32_t* n_valid, uint16_t* dlogits, int64_t ld_d, void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 31) || V < 1 || V >= ((int64_t)1 << 40) || ld < V || ld % 8 ||
      ld_d < V || ld_d % 8)
    return QLORA_ESHAPE;
  if (m == 0) return QLORA_OK;
  if (!logits || !labels || !lse || !n_valid || !dlogits) return QLORA_EINVAL;
  if (logits == dlogits && ld != ld_d) return QLORA_EINVAL;   // in place only with the same pitch
  if (!al16(logits) || !al16(dlogits) || ((uintptr_t)labels & 7) || ((uintptr_t)lse & 3) ||
      ((uintptr_t)n_valid & 3) || ((uintptr_t)dloss & 3))
    return QLORA_ESHAPE;
  QL_TRY(launch_xent_bwd(logits, ld, m, V, labels, lse, dloss, n_valid, dlogits, ld_d,
                         (hipStream_t)stream),
         "cross_entropy_bwd");
  return QLORA_OK;
}

int qlora_cross_entropy_fused(const uint16_t* logits, int64_t ld, int64_t m, int64_t V,
                              const int64_t* labels, float dloss, float* lse, float* ce_rows,
                              float* loss, int32_t* n_valid, uint16_t* dlogits, int64_t ld_d,
                              void* stream) {
  if (m < 0 || m >= ((int64_t)1 << 31) || V < 1 || V >= ((int64_t)1 << 40) || ld < V || ld % 8 ||
      ld_d < V || ld_d % 8)
    return QLORA_ESHAPE;
  if (!loss || !n_valid || !std::isfinite(dloss)) return QLORA_EINVAL;
  if (m > 0 && (!logits || !labels || !lse || !ce_rows || !dlogits)) return QLORA_EINVAL;
  if (m > 0 && logits == dlogits && ld != ld_d) return QLORA_EINVAL;
  if (m > 0 && (!al16(logits) || !al16(dlogits) || ((uintptr_t)labels & 7) ||
                ((uintptr_t)lse & 3) || ((uintptr_t)ce_rows & 3)))
    return QLORA_ESHAPE;
  if (((uintptr_t)loss & 3) || ((uintptr_t)n_valid & 3)) return QLORA_ESHAPE;
  QL_TRY(launch_xent_fused(logits, ld, m, V, labels, dloss, lse, ce_rows, loss, n_valid, dlogits, ld_d,
                           (hipStream_t)stream),
         "cross_entropy_fused");
  return QLORA_OK;
}

}  // extern "C"
