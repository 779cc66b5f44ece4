// sage_api.cpp -- the C ABI declared in include/sage.h: argument checks, workspace
// layout, dispatch to the gfx950 kernels.  Every check runs before any HIP call, so a
// rejected call touches neither the GPU nor the HIP runtime.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sage.h"
#include "sage_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SAGE_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SAGE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kPad = 128;

int pad_len(int N) { return (N + kPad - 1) / kPad * kPad; }
int ceil_div(int a, int b) { return (a + b - 1) / b; }
bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

struct Params {
  int blk_q = 128, blk_k = 64, smooth_k = 1, smooth_q = 0, smooth_v = 0;
  int q_group = 0;  // rows per Q scale; resolved to blk_q when 0
};

// Earlier layouts of sage_params: five ints (library 0.1), six ints (0.2, + smooth_v).
constexpr int kParamsV1Size = 5 * (int)sizeof(int), kParamsV2Size = 6 * (int)sizeof(int);

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int read_params(const sage_params* p, int variant, Params* out) {
  Params r;
  r.smooth_q = variant == SAGE_VARIANT_INT8QK_FP8PV ? 1 : 0;
  if (p) {
    if (p->struct_size != (int)sizeof(sage_params) && p->struct_size != kParamsV1Size &&
        p->struct_size != kParamsV2Size)
      return fail(SAGE_ERR_INVALID_ARG, "sage_params.struct_size must be %d", (int)sizeof(sage_params));
    r.blk_q = p->blk_q;
    r.blk_k = p->blk_k;
    r.smooth_k = p->smooth_k;
    r.smooth_q = p->smooth_q;
    if (p->struct_size >= kParamsV2Size) r.smooth_v = p->smooth_v;
    if (p->struct_size >= (int)sizeof(sage_params)) r.q_group = p->q_group;
  }
  if (r.blk_q != 32 && r.blk_q != 64 && r.blk_q != 128)
    return fail(SAGE_ERR_UNSUPPORTED, "blk_q must be 32, 64 or 128 (got %d)", r.blk_q);
  if (r.blk_k != 16 && r.blk_k != 32 && r.blk_k != 64 && r.blk_k != 128)
    return fail(SAGE_ERR_UNSUPPORTED, "blk_k must be 16, 32, 64 or 128 (got %d)", r.blk_k);
  if ((r.smooth_k != 0 && r.smooth_k != 1) || (r.smooth_q != 0 && r.smooth_q != 1) ||
      (r.smooth_v != 0 && r.smooth_v != 1))
    return fail(SAGE_ERR_INVALID_ARG, "smooth_k / smooth_q / smooth_v must be 0 or 1");
  if (r.smooth_v && variant == SAGE_VARIANT_INT8QK_FP16PV)
    return fail(SAGE_ERR_UNSUPPORTED, "smooth_v applies to the FP8 / FP4 P~V variants only");
  if (r.smooth_q && (variant == SAGE_VARIANT_MXFP4QK_FP8PV || variant == SAGE_VARIANT_MXFP4QK_FP4PV))
    return fail(SAGE_ERR_UNSUPPORTED, "the MXFP4 variants quantise Q per token without smoothing (smooth_q must be 0)");
  if (r.q_group == 0) r.q_group = r.blk_q;
  if (!pow2(r.q_group) || r.q_group > r.blk_q)
    return fail(SAGE_ERR_UNSUPPORTED, "q_group must be 0 or a power of two <= blk_q (got %d)", r.q_group);
  *out = r;
  return SAGE_OK;
}

int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return fail(SAGE_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (d != 64 && d != 128) return fail(SAGE_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %d)", d);
  const long long elems = (long long)B * H * pad_len(N) * d;
  if (elems >= (1LL << 31)) return fail(SAGE_ERR_INVALID_ARG, "B*H*pad_len(N)*d must be < 2^31");
  return SAGE_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(SAGE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(SAGE_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return SAGE_OK;
}

// The whole call quantises Q inside the attention kernel for every variant (INT8 with or
// without Q smoothing, MXFP4); the pre-quantised entry points read the quantisation pass's Q.
bool fuse_q(int variant, const Params& p) {
  (void)variant;
  (void)p;
  return true;
}

bool valid_variant(int variant) { return variant >= 0 && variant <= 3; }

// Workspace layout (each piece 256-byte aligned).  Variants 2 and 3 keep their packed
// E2M1 codes in q_i8 / k_i8 (d/2 bytes per row) and their E8M0 scales in q_e8 / k_e8;
// variant 3 keeps V's E2M1 pairs in v_f8 (d rows of Np/2 bytes) and its scales in v_e8.
struct Layout {
  size_t ksum, vsum, vmax, vmin, q_i8, k_i8, q_scale, k_scale, k_mean, q_mean, v_f8, v_scale, v_mean, q_e8, k_e8,
      v_e8, total;
};

size_t up(size_t x) { return (x + 255) / 256 * 256; }

Layout layout(int B, int H, int N, int d, int variant, const Params& p) {
  const size_t G = (size_t)B * H, Np = pad_len(N), ns = ceil_div(N, sage::kStatRows);
  const size_t nqb = ceil_div(N, p.blk_q), nkb = ceil_div(N, p.blk_k), nqg = ceil_div(N, p.q_group);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes); return o; };
  const bool fp8v = variant != 0, mx = variant >= 2, v4 = variant == 3;
  L.ksum = take(G * ns * d * sizeof(long long));
  L.vsum = take(fp8v ? G * ns * d * sizeof(long long) : 0);
  L.vmax = take(fp8v ? G * ns * d * sizeof(float) : 0);
  L.vmin = take(fp8v ? G * ns * d * sizeof(float) : 0);
  const bool fq = fuse_q(variant, p);
  L.q_i8 = take(fq ? 0 : G * Np * (mx ? d / 2 : d));
  L.k_i8 = take(G * Np * (mx ? d / 2 : d));
  L.q_scale = take(fq || mx ? 0 : G * nqg * sizeof(float));
  L.k_scale = take(mx ? 0 : G * nkb * sizeof(float));
  L.k_mean = take(G * d * sizeof(float));
  L.q_mean = take(p.smooth_q && !fq ? G * nqb * d * sizeof(float) : 0);
  L.v_f8 = take(fp8v ? G * d * (v4 ? Np / 2 : Np) : 0);
  L.v_scale = take(fp8v && !v4 ? G * d * sizeof(float) : 0);
  L.v_mean = take(p.smooth_v ? G * d * sizeof(float) : 0);
  L.q_e8 = take(mx && !fq ? G * Np * (d / 32) : 0);
  L.k_e8 = take(mx ? G * Np * (d / 32) : 0);
  L.v_e8 = take(v4 ? G * (Np / 32) * d : 0);
  L.total = off;
  return L;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SAGE_OK;
  if (!ws) return fail(SAGE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(SAGE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(SAGE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return SAGE_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

sage::QuantArgs quant_args(const void* q, const void* k, int B, int H, int N, int d, const Params& p, int8_t* q_i8,
                           int8_t* k_i8, float* q_scale, float* k_scale, float* k_mean, float* q_mean,
                           const long long* ksum) {
  (void)d;
  sage::QuantArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.q_i8 = q_i8;
  a.k_i8 = k_i8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.k_mean = k_mean;
  a.q_mean = q_mean;
  a.ksum_part = ksum;
  a.G = B * H;
  a.N = N;
  a.Np = pad_len(N);
  a.blk_q = p.blk_q;
  a.blk_k = p.blk_k;
  a.nqb = ceil_div(N, p.blk_q);
  a.nkb = ceil_div(N, p.blk_k);
  a.nsplit = ceil_div(N, sage::kStatRows);
  a.smooth_k = p.smooth_k;
  a.smooth_q = p.smooth_q;
  a.q_group = p.q_group;
  a.nqg = ceil_div(N, p.q_group);
  a.with_q = 1;
  return a;
}

sage::AttnArgs attn_args(int B, int H, int N, const Params& p, float sm_scale) {
  sage::AttnArgs a{};
  a.G = B * H;
  a.N = N;
  a.Np = pad_len(N);
  a.blk_q = p.blk_q;
  a.blk_k = p.blk_k;
  a.nqb = ceil_div(N, p.blk_q);
  a.nkb = ceil_div(N, p.blk_k);
  a.q_group = p.q_group;
  a.nqg = ceil_div(N, p.q_group);
  a.kscale = sm_scale * 1.4426950408889634f;
  return a;
}

int run_quant_qk(const void* q, const void* k, int B, int H, int N, int d, const Params& p, int8_t* q_i8,
                 int8_t* k_i8, float* q_scale, float* k_scale, float* k_mean, float* q_mean, long long* ksum,
                 hipStream_t st) {
  hipError_t e;
  if (p.smooth_k) {
    e = sage::launch_stats(d, k, nullptr, false, B * H, N, sage::StatsOut{ksum, nullptr, nullptr, nullptr}, st);
    if (e != hipSuccess) return hip_fail(e, "statistics kernel");
  }
  e = sage::launch_quant(d, quant_args(q, k, B, H, N, d, p, q_i8, k_i8, q_scale, k_scale, k_mean, q_mean, ksum), st);
  if (e != hipSuccess) return hip_fail(e, "quantisation kernel");
  return SAGE_OK;
}

int attn_common(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int causal,
                float sm_scale, int variant, const sage_params* pp, void* ws, size_t ws_bytes, void* stream,
                float* lse = nullptr) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!valid_variant(variant)) return fail(SAGE_ERR_INVALID_ARG, "variant must be 0, 1, 2 or 3");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, variant, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k, 16, "k")) || (rc = check_ptr(v, 16, "v")) ||
      (rc = check_ptr(o, 16, "o")))
    return rc;
  const Layout L = layout(B, H, N, d, variant, p);
  if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;

  hipStream_t st = (hipStream_t)stream;
  const int G = B * H, Np = pad_len(N);
  hipError_t e;
  const sage::StatsOut stats{at<long long>(ws, L.ksum), at<long long>(ws, L.vsum), at<float>(ws, L.vmax),
                             at<float>(ws, L.vmin)};
  if (p.smooth_k || variant != 0) {
    e = sage::launch_stats(d, k, variant != 0 ? v : nullptr, p.smooth_v, G, N, stats, st);
    if (e != hipSuccess) return hip_fail(e, "statistics kernel");
  }
  const bool fq = fuse_q(variant, p);
  if (variant >= 2) {
    // (Q is quantised by the attention kernel itself)
    e = sage::launch_quant_mx(d, k, G, N, Np, at<long long>(ws, L.ksum), p.smooth_k, at<uint8_t>(ws, L.k_i8),
                              at<uint8_t>(ws, L.k_e8), at<float>(ws, L.k_mean), st);
    if (e != hipSuccess) return hip_fail(e, "MXFP4 quantisation kernel");
  } else {
    sage::QuantArgs qa = quant_args(q, k, B, H, N, d, p, fq ? nullptr : at<int8_t>(ws, L.q_i8),
                                    at<int8_t>(ws, L.k_i8), fq ? nullptr : at<float>(ws, L.q_scale),
                                    at<float>(ws, L.k_scale), at<float>(ws, L.k_mean),
                                    p.smooth_q && !fq ? at<float>(ws, L.q_mean) : nullptr, at<long long>(ws, L.ksum));
    qa.with_q = fq ? 0 : 1;
    e = sage::launch_quant(d, qa, st);
    if (e != hipSuccess) return hip_fail(e, "quantisation kernel");
  }
  if (variant == 3) {
    e = sage::launch_quant_v_mx(d, v, G, N, Np, stats.vsum, p.smooth_v, at<uint8_t>(ws, L.v_f8),
                                at<uint8_t>(ws, L.v_e8), p.smooth_v ? at<float>(ws, L.v_mean) : nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "MXFP4 V quantisation kernel");
  } else if (variant != 0) {
    e = sage::launch_quant_v(d, v, G, N, Np, stats, p.smooth_v, at<uint8_t>(ws, L.v_f8), at<float>(ws, L.v_scale),
                             p.smooth_v ? at<float>(ws, L.v_mean) : nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "V quantisation kernel");
  }
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q = fq ? (const uint16_t*)q : nullptr;
  a.q_i8 = fq ? nullptr : at<int8_t>(ws, L.q_i8);
  a.k_i8 = at<int8_t>(ws, L.k_i8);
  a.q_scale = fq || variant >= 2 ? nullptr : at<float>(ws, L.q_scale);
  a.k_scale = variant >= 2 ? nullptr : at<float>(ws, L.k_scale);
  a.q_mean = p.smooth_q && !fq ? at<float>(ws, L.q_mean) : nullptr;
  a.q_e8 = nullptr;  // variants 2 and 3 quantise Q in the kernel
  a.k_e8 = variant >= 2 ? at<uint8_t>(ws, L.k_e8) : nullptr;
  a.v = (const uint16_t*)v;
  a.v_f8 = variant != 0 ? at<uint8_t>(ws, L.v_f8) : nullptr;
  a.v_e8 = variant == 3 ? at<uint8_t>(ws, L.v_e8) : nullptr;
  a.v_scale = variant == 1 || variant == 2 ? at<float>(ws, L.v_scale) : nullptr;
  a.v_mean = p.smooth_v ? at<float>(ws, L.v_mean) : nullptr;
  a.o = (uint16_t*)o;
  a.lse = lse;
  e = sage::launch_attn(d, variant, causal, p.smooth_q, a, st);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

// Backward workspace (each piece 256-byte aligned).
struct BwdLayout {
  size_t ksum, vsum, vmax, vmin, q_i8, k_i8, q_scale, k_scale, k_mean, v_i8, do_i8, v_scale, do_scale, dvec, lse2,
      nrm, kp, total;
};

BwdLayout bwd_layout(int B, int H, int N, int d, const Params& p) {
  const size_t G = (size_t)B * H, Np = pad_len(N), ns = ceil_div(N, sage::kStatRows);
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes); return o; };
  L.ksum = take(G * ns * d * sizeof(long long));
  L.vsum = take(G * ns * d * sizeof(long long));
  L.vmax = take(G * ns * d * sizeof(float));
  L.vmin = take(G * ns * d * sizeof(float));
  L.q_i8 = take(G * Np * d);
  L.k_i8 = take(G * Np * d);
  L.q_scale = take(G * ceil_div(N, p.blk_q) * sizeof(float));
  L.k_scale = take(G * ceil_div(N, p.blk_k) * sizeof(float));
  L.k_mean = take(G * d * sizeof(float));
  L.v_i8 = take(G * Np * d);
  L.do_i8 = take(G * Np * d);
  L.v_scale = take(G * Np * sizeof(float));
  L.do_scale = take(G * Np * sizeof(float));
  L.dvec = take(G * Np * sizeof(float));
  L.lse2 = take(G * Np * sizeof(float));
  L.nrm = take(G * (Np / 64) * 2 * sizeof(float));
  L.kp = take(G * Np * d * sizeof(uint16_t));
  L.total = off;
  return L;
}

// The backward differentiates the variant-0 forward: per-block Q scales of 64 or 128 rows
// (a 64-row query tile lies in one block), no Q smoothing, one Q scale per block.
int read_bwd_params(const sage_params* pp, Params* p) {
  int rc;
  if ((rc = read_params(pp, SAGE_VARIANT_INT8QK_FP16PV, p))) return rc;
  if (p->blk_q < 64) return fail(SAGE_ERR_UNSUPPORTED, "the backward needs blk_q = 64 or 128 (got %d)", p->blk_q);
  if (p->smooth_q) return fail(SAGE_ERR_UNSUPPORTED, "the backward differentiates the forward without Q smoothing");
  if (p->q_group != p->blk_q) return fail(SAGE_ERR_UNSUPPORTED, "the backward takes one Q scale per block (q_group = 0)");
  return SAGE_OK;
}

// Workspace of sage_attn_fwd_noalloc: one array per GPU, held for the life of the process.
// Host code never uses the array's name as an address: on the host it is only a handle,
// and its device address comes from hipGetSymbolAddress (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per device with
// that device current.  Returns SAGE_OK and sets *out, or an error status.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SAGE_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(SAGE_ERR_HIP, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SAGE_OK;
}

}  // namespace

extern "C" {

int sage_version(void) { return 400; }

int sage_pad_len(int N) { return N < 1 ? -1 : pad_len(N); }

int sage_kv_tile(int variant, int d) {
  if (!valid_variant(variant) || (d != 64 && d != 128)) return -1;
  return 64;
}

size_t sage_workspace_bytes(int B, int H, int N, int d, int variant, const sage_params* pp) {
  if (check_shape(B, H, N, d) || !valid_variant(variant)) return 0;
  Params p;
  if (read_params(pp, variant, &p)) return 0;
  return layout(B, H, N, d, variant, p).total;
}

int sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d, const sage_params* pp, int8_t* q_i8,
                  int8_t* k_i8, float* q_scale, float* k_scale, float* k_mean, float* q_mean, void* ws,
                  size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  Params p;
  if ((rc = read_params(pp, 0, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k, 16, "k")) || (rc = check_ptr(q_i8, 16, "q_i8")) ||
      (rc = check_ptr(k_i8, 16, "k_i8")) || (rc = check_ptr(q_scale, 4, "q_scale")) ||
      (rc = check_ptr(k_scale, 4, "k_scale")))
    return rc;
  if (k_mean && !aligned(k_mean, 4)) return fail(SAGE_ERR_INVALID_ARG, "k_mean must be 4-byte aligned");
  if (p.smooth_q && (rc = check_ptr(q_mean, 4, "q_mean (required with smooth_q)"))) return rc;
  const size_t need = p.smooth_k ? up((size_t)B * H * ceil_div(N, sage::kStatRows) * d * sizeof(long long)) : 0;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  rc = run_quant_qk(q, k, B, H, N, d, p, q_i8, k_i8, q_scale, k_scale, k_mean, p.smooth_q ? q_mean : nullptr,
                    (long long*)ws, (hipStream_t)stream);
  return rc ? rc : ok();
}

int sage_quant_v_ex(const void* v, int B, int H, int N, int d, int smooth_v, uint8_t* v_f8, float* v_scale,
                    float* v_mean, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (smooth_v != 0 && smooth_v != 1) return fail(SAGE_ERR_INVALID_ARG, "smooth_v must be 0 or 1");
  if ((rc = check_ptr(v, 16, "v")) || (rc = check_ptr(v_f8, 16, "v_f8")) || (rc = check_ptr(v_scale, 16, "v_scale")))
    return rc;
  if (smooth_v && (rc = check_ptr(v_mean, 16, "v_mean (required with smooth_v)"))) return rc;
  const size_t G = (size_t)B * H, ns = ceil_div(N, sage::kStatRows);
  const size_t i64 = up(G * ns * d * sizeof(long long)), f32 = up(G * ns * d * sizeof(float));
  if ((rc = check_ws(ws, ws_bytes, 2 * i64 + 2 * f32))) return rc;
  hipStream_t st = (hipStream_t)stream;
  const sage::StatsOut stats{at<long long>(ws, 0), at<long long>(ws, i64), at<float>(ws, 2 * i64),
                             at<float>(ws, 2 * i64 + f32)};
  // the statistics pass reads K and V together; with V as "K" too the K sums are unused
  hipError_t e = sage::launch_stats(d, v, v, smooth_v, (int)G, N, stats, st);
  if (e != hipSuccess) return hip_fail(e, "statistics kernel");
  e = sage::launch_quant_v(d, v, (int)G, N, pad_len(N), stats, smooth_v, v_f8, v_scale, smooth_v ? v_mean : nullptr,
                           st);
  if (e != hipSuccess) return hip_fail(e, "V quantisation kernel");
  return ok();
}

int sage_quant_v(const void* v, int B, int H, int N, int d, uint8_t* v_f8, float* v_scale, void* ws,
                 size_t ws_bytes, void* stream) {
  return sage_quant_v_ex(v, B, H, N, d, 0, v_f8, v_scale, nullptr, ws, ws_bytes, stream);
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int causal,
                  float sm_scale, int variant, void* ws, size_t ws_bytes, void* stream) {
  return attn_common(q, k, v, o, B, H, N, d, causal, sm_scale, variant, nullptr, ws, ws_bytes, stream);
}

int sage_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, int causal,
                     float sm_scale, int variant, const sage_params* p, void* ws, size_t ws_bytes, void* stream) {
  return attn_common(q, k, v, o, B, H, N, d, causal, sm_scale, variant, p, ws, ws_bytes, stream);
}

int sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                          int causal, float sm_scale, int variant, const sage_params* pp, void* stream) {
  int rc;
  // the argument checks of sage_attn_fwd_ex, then the size check, before any HIP call
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (!valid_variant(variant)) return fail(SAGE_ERR_INVALID_ARG, "variant must be 0, 1, 2 or 3");
  Params p;
  if ((rc = read_params(pp, variant, &p))) return rc;
  const size_t need = layout(B, H, N, d, variant, p).total;
  if (need > (size_t)SAGE_NOALLOC_SCRATCH_BYTES)
    return fail(SAGE_ERR_WORKSPACE, "this shape needs %zu bytes of workspace; sage_attn_fwd_noalloc has %zu",
                need, (size_t)SAGE_NOALLOC_SCRATCH_BYTES);
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k, 16, "k")) || (rc = check_ptr(v, 16, "v")) ||
      (rc = check_ptr(o, 16, "o")))
    return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return attn_common(q, k, v, o, B, H, N, d, causal, sm_scale, variant, pp, ws, (size_t)SAGE_NOALLOC_SCRATCH_BYTES,
                     stream);
}

int sage_attn_fwd_train(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                        int d, int causal, float sm_scale, const sage_params* pp, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc;
  Params p;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if ((rc = read_bwd_params(pp, &p))) return rc;
  if ((rc = check_ptr(lse, 16, "lse"))) return rc;
  return attn_common(q, k, v, o, B, H, N, d, causal, sm_scale, SAGE_VARIANT_INT8QK_FP16PV, pp, ws, ws_bytes, stream,
                     lse);
}

size_t sage_attn_bwd_workspace_bytes(int B, int H, int N, int d, const sage_params* pp) {
  if (check_shape(B, H, N, d)) return 0;
  Params p;
  if (read_bwd_params(pp, &p)) return 0;
  return bwd_layout(B, H, N, d, p).total;
}

int sage_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  float* dq, float* dk, float* dv, int B, int H, int N, int d, int causal, float sm_scale,
                  const sage_params* pp, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_bwd_params(pp, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k, 16, "k")) || (rc = check_ptr(v, 16, "v")) ||
      (rc = check_ptr(o, 16, "o")) || (rc = check_ptr(dout, 16, "dout")) || (rc = check_ptr(lse, 16, "lse")) ||
      (rc = check_ptr(dq, 16, "dq")) || (rc = check_ptr(dk, 16, "dk")) || (rc = check_ptr(dv, 16, "dv")))
    return rc;
  const BwdLayout L = bwd_layout(B, H, N, d, p);
  if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int G = B * H;
  // exact token sums of K and V (the V sums give V's mean for the smoothed dP)
  const sage::StatsOut stats{at<long long>(ws, L.ksum), at<long long>(ws, L.vsum), at<float>(ws, L.vmax),
                             at<float>(ws, L.vmin)};
  hipError_t e = sage::launch_stats(d, k, v, true, G, N, stats, st);
  if (e != hipSuccess) return hip_fail(e, "statistics kernel");
  // the forward's codes: variant 0, K smoothed, per-block Q and K scales
  sage::QuantArgs qa = quant_args(q, k, B, H, N, d, p, at<int8_t>(ws, L.q_i8), at<int8_t>(ws, L.k_i8),
                                  at<float>(ws, L.q_scale), at<float>(ws, L.k_scale), at<float>(ws, L.k_mean), nullptr,
                                  at<long long>(ws, L.ksum));
  e = sage::launch_quant(d, qa, st);
  if (e != hipSuccess) return hip_fail(e, "quantisation kernel");
  sage::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.q_i8 = at<int8_t>(ws, L.q_i8);
  a.k_i8 = at<int8_t>(ws, L.k_i8);
  a.q_scale = at<float>(ws, L.q_scale);
  a.k_scale = at<float>(ws, L.k_scale);
  a.ksum = at<long long>(ws, L.ksum);
  a.vsum = at<long long>(ws, L.vsum);
  a.v_i8 = at<int8_t>(ws, L.v_i8);
  a.do_i8 = at<int8_t>(ws, L.do_i8);
  a.v_scale = at<float>(ws, L.v_scale);
  a.do_scale = at<float>(ws, L.do_scale);
  a.dvec = at<float>(ws, L.dvec);
  a.lse2 = at<float>(ws, L.lse2);
  a.nrm = at<float>(ws, L.nrm);
  a.kp = at<uint16_t>(ws, L.kp);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.G = G;
  a.N = N;
  a.Np = pad_len(N);
  a.blk_q = p.blk_q;
  a.blk_k = p.blk_k;
  a.nqb = ceil_div(N, p.blk_q);
  a.nkb = ceil_div(N, p.blk_k);
  a.nsplit = ceil_div(N, sage::kStatRows);
  a.smooth_k = p.smooth_k;
  a.kscale = sm_scale * 1.4426950408889634f;
  a.sm_scale = sm_scale;
  e = sage::launch_bwd(d, causal, a, st);
  if (e != hipSuccess) return hip_fail(e, "backward kernels");
  return ok();
}

int sage_attn_fwd_prequant(const int8_t* q_i8, const int8_t* k_i8, const float* q_scale, const float* k_scale,
                           const float* q_mean, const void* v, const uint8_t* v_f8, const float* v_scale,
                           const float* v_mean, void* o, int B, int H, int N, int d, int causal, float sm_scale,
                           int variant, const sage_params* pp, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (variant != 0 && variant != 1)
    return fail(SAGE_ERR_INVALID_ARG, "variant must be 0 or 1 (the MXFP4 variant: sage_attn_fwd_prequant_mx)");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, variant, &p))) return rc;
  if ((rc = check_ptr(q_i8, 16, "q_i8")) || (rc = check_ptr(k_i8, 16, "k_i8")) ||
      (rc = check_ptr(q_scale, 4, "q_scale")) || (rc = check_ptr(k_scale, 4, "k_scale")) ||
      (rc = check_ptr(o, 16, "o")))
    return rc;
  if (variant == 0 && (rc = check_ptr(v, 16, "v"))) return rc;
  if (variant == 1 && ((rc = check_ptr(v_f8, 16, "v_f8")) || (rc = check_ptr(v_scale, 16, "v_scale")))) return rc;
  if (p.smooth_q && (rc = check_ptr(q_mean, 4, "q_mean (required with smooth_q)"))) return rc;
  if (p.smooth_v && (rc = check_ptr(v_mean, 16, "v_mean (required with smooth_v)"))) return rc;
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q_i8 = q_i8;
  a.k_i8 = k_i8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.q_mean = q_mean;
  a.v = (const uint16_t*)v;
  a.v_f8 = v_f8;
  a.v_scale = v_scale;
  a.v_mean = p.smooth_v ? v_mean : nullptr;
  a.o = (uint16_t*)o;
  hipError_t e = sage::launch_attn(d, variant, causal, p.smooth_q, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

int sage_attn_fwd_qf16(const void* q, const int8_t* k_i8, const float* k_scale, const void* v, void* o, int B,
                       int H, int N, int d, int causal, float sm_scale, const sage_params* pp, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, 0, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k_i8, 16, "k_i8")) || (rc = check_ptr(k_scale, 4, "k_scale")) ||
      (rc = check_ptr(v, 16, "v")) || (rc = check_ptr(o, 16, "o")))
    return rc;
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q = (const uint16_t*)q;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  hipError_t e = sage::launch_attn(d, 0, causal, p.smooth_q, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

int sage_attn_fwd_qf16_fp8(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_f8,
                           const float* v_scale, const float* v_mean, void* o, int B, int H, int N, int d, int causal,
                           float sm_scale, const sage_params* pp, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, SAGE_VARIANT_INT8QK_FP8PV, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k_i8, 16, "k_i8")) || (rc = check_ptr(k_scale, 4, "k_scale")) ||
      (rc = check_ptr(v_f8, 16, "v_f8")) || (rc = check_ptr(v_scale, 16, "v_scale")) || (rc = check_ptr(o, 16, "o")))
    return rc;
  if (p.smooth_v && (rc = check_ptr(v_mean, 16, "v_mean (required with smooth_v)"))) return rc;
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q = (const uint16_t*)q;
  a.k_i8 = k_i8;
  a.k_scale = k_scale;
  a.v_f8 = v_f8;
  a.v_scale = v_scale;
  a.v_mean = p.smooth_v ? v_mean : nullptr;
  a.o = (uint16_t*)o;
  hipError_t e = sage::launch_attn(d, 1, causal, p.smooth_q, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

int sage_quant_qk_mx(const void* q, const void* k, int B, int H, int N, int d, int smooth_k, uint8_t* q_f4,
                     uint8_t* k_f4, uint8_t* q_e8, uint8_t* k_e8, float* k_mean, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (smooth_k != 0 && smooth_k != 1) return fail(SAGE_ERR_INVALID_ARG, "smooth_k must be 0 or 1");
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k, 16, "k")) || (rc = check_ptr(q_f4, 16, "q_f4")) ||
      (rc = check_ptr(k_f4, 16, "k_f4")) || (rc = check_ptr(q_e8, 4, "q_e8")) || (rc = check_ptr(k_e8, 4, "k_e8")))
    return rc;
  if (k_mean && !aligned(k_mean, 4)) return fail(SAGE_ERR_INVALID_ARG, "k_mean must be 4-byte aligned");
  const size_t need = smooth_k ? up((size_t)B * H * ceil_div(N, sage::kStatRows) * d * sizeof(long long)) : 0;
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int G = B * H, Np = pad_len(N);
  hipError_t e = hipSuccess;
  if (smooth_k)
    e = sage::launch_stats(d, k, nullptr, false, G, N, sage::StatsOut{(long long*)ws, nullptr, nullptr, nullptr}, st);
  if (e != hipSuccess) return hip_fail(e, "statistics kernel");
  e = sage::launch_quant_mx(d, k, G, N, Np, (const long long*)ws, smooth_k, k_f4, k_e8, k_mean, st);
  if (e == hipSuccess) e = sage::launch_quant_mx(d, q, G, N, Np, nullptr, 0, q_f4, q_e8, nullptr, st);
  if (e != hipSuccess) return hip_fail(e, "MXFP4 quantisation kernel");
  return ok();
}

int sage_attn_fwd_prequant_mx(const uint8_t* q_f4, const uint8_t* k_f4, const uint8_t* q_e8, const uint8_t* k_e8,
                              const uint8_t* v_f8, const float* v_scale, const float* v_mean, void* o, int B, int H,
                              int N, int d, int causal, float sm_scale, const sage_params* pp, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, SAGE_VARIANT_MXFP4QK_FP8PV, &p))) return rc;
  if ((rc = check_ptr(q_f4, 16, "q_f4")) || (rc = check_ptr(k_f4, 16, "k_f4")) || (rc = check_ptr(q_e8, 4, "q_e8")) ||
      (rc = check_ptr(k_e8, 4, "k_e8")) || (rc = check_ptr(v_f8, 16, "v_f8")) ||
      (rc = check_ptr(v_scale, 16, "v_scale")) || (rc = check_ptr(o, 16, "o")))
    return rc;
  if (p.smooth_v && (rc = check_ptr(v_mean, 16, "v_mean (required with smooth_v)"))) return rc;
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q_i8 = (const int8_t*)q_f4;
  a.k_i8 = (const int8_t*)k_f4;
  a.q_e8 = q_e8;
  a.k_e8 = k_e8;
  a.v_f8 = v_f8;
  a.v_scale = v_scale;
  a.v_mean = p.smooth_v ? v_mean : nullptr;
  a.o = (uint16_t*)o;
  hipError_t e = sage::launch_attn(d, 2, causal, 0, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

int sage_attn_fwd_qf16_mx(const void* q, const uint8_t* k_f4, const uint8_t* k_e8, const uint8_t* v_f8,
                          const float* v_scale, const float* v_mean, void* o, int B, int H, int N, int d, int causal,
                          float sm_scale, const sage_params* pp, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, SAGE_VARIANT_MXFP4QK_FP8PV, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k_f4, 16, "k_f4")) || (rc = check_ptr(k_e8, 4, "k_e8")) ||
      (rc = check_ptr(v_f8, 16, "v_f8")) || (rc = check_ptr(v_scale, 16, "v_scale")) || (rc = check_ptr(o, 16, "o")))
    return rc;
  if (p.smooth_v && (rc = check_ptr(v_mean, 16, "v_mean (required with smooth_v)"))) return rc;
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q = (const uint16_t*)q;
  a.k_i8 = (const int8_t*)k_f4;
  a.k_e8 = k_e8;
  a.v_f8 = v_f8;
  a.v_scale = v_scale;
  a.v_mean = p.smooth_v ? v_mean : nullptr;
  a.o = (uint16_t*)o;
  hipError_t e = sage::launch_attn(d, 2, causal, 0, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

int sage_quant_v_mx(const void* v, int B, int H, int N, int d, int smooth_v, uint8_t* v_f4, uint8_t* v_e8,
                    float* v_mean, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (smooth_v != 0 && smooth_v != 1) return fail(SAGE_ERR_INVALID_ARG, "smooth_v must be 0 or 1");
  if ((rc = check_ptr(v, 16, "v")) || (rc = check_ptr(v_f4, 16, "v_f4")) || (rc = check_ptr(v_e8, 4, "v_e8")))
    return rc;
  if (smooth_v && (rc = check_ptr(v_mean, 4, "v_mean (required with smooth_v)"))) return rc;
  const size_t G = (size_t)B * H, ns = ceil_div(N, sage::kStatRows);
  const size_t i64 = up(G * ns * d * sizeof(long long)), f32 = up(G * ns * d * sizeof(float));
  hipStream_t st = (hipStream_t)stream;
  if (smooth_v) {
    // the token sums of V from the statistics pass (V given as K too; its K sums go unused)
    if ((rc = check_ws(ws, ws_bytes, 2 * i64 + 2 * f32))) return rc;
    const sage::StatsOut stats{at<long long>(ws, 0), at<long long>(ws, i64), at<float>(ws, 2 * i64),
                               at<float>(ws, 2 * i64 + f32)};
    hipError_t e = sage::launch_stats(d, v, v, true, (int)G, N, stats, st);
    if (e != hipSuccess) return hip_fail(e, "statistics kernel");
  }
  hipError_t e = sage::launch_quant_v_mx(d, v, (int)G, N, pad_len(N), smooth_v ? at<long long>(ws, i64) : nullptr,
                                         smooth_v, v_f4, v_e8, smooth_v ? v_mean : nullptr, st);
  if (e != hipSuccess) return hip_fail(e, "MXFP4 V quantisation kernel");
  return ok();
}

int sage_attn_fwd_qf16_fp4(const void* q, const uint8_t* k_f4, const uint8_t* k_e8, const uint8_t* v_f4,
                           const uint8_t* v_e8, const float* v_mean, void* o, int B, int H, int N, int d, int causal,
                           float sm_scale, const sage_params* pp, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale))
    return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  Params p;
  if ((rc = read_params(pp, SAGE_VARIANT_MXFP4QK_FP4PV, &p))) return rc;
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k_f4, 16, "k_f4")) || (rc = check_ptr(k_e8, 4, "k_e8")) ||
      (rc = check_ptr(v_f4, 16, "v_f4")) || (rc = check_ptr(v_e8, 4, "v_e8")) || (rc = check_ptr(o, 16, "o")))
    return rc;
  if (p.smooth_v && (rc = check_ptr(v_mean, 16, "v_mean (required with smooth_v)"))) return rc;
  sage::AttnArgs a = attn_args(B, H, N, p, sm_scale);
  a.q = (const uint16_t*)q;
  a.k_i8 = (const int8_t*)k_f4;
  a.k_e8 = k_e8;
  a.v_f8 = v_f4;
  a.v_e8 = v_e8;
  a.v_mean = p.smooth_v ? v_mean : nullptr;
  a.o = (uint16_t*)o;
  hipError_t e = sage::launch_attn(d, 3, causal, 0, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return ok();
}

int sage_debug_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d, const int* tiles,
                        int n_tiles, int32_t* s_out, void* stream) {
  int rc;
  if ((rc = check_shape(B, H, N, d))) return rc;
  if (n_tiles < 1) return fail(SAGE_ERR_INVALID_ARG, "n_tiles must be >= 1");
  if ((rc = check_ptr(q_i8, 16, "q_i8")) || (rc = check_ptr(k_i8, 16, "k_i8")) || (rc = check_ptr(tiles, 4, "tiles")) ||
      (rc = check_ptr(s_out, 16, "s_out")))
    return rc;
  hipError_t e = sage::launch_debug_qk(d, q_i8, k_i8, B * H, pad_len(N), tiles, n_tiles, s_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug QK kernel");
  return ok();
}

const char* sage_last_error(void) { return g_err; }

}  // extern "C"
