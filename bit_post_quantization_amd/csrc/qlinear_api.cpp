// C ABI of libqlinear.so (declared in include/qlinear.h): argument checks,
// the plan object, and the launches of the HIP kernels on the caller's
// stream. No computation of the method happens here.
#include "../../include/qlinear.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "ql_kernels.h"

namespace {
// Device buffer shared by a plan and its TASQ views (freed with the last).
using DevBuf = std::shared_ptr<uint8_t>;

hipError_t dev_alloc(DevBuf& out, size_t bytes) {
  void* p = nullptr;
  const hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) return e;
  out = DevBuf(static_cast<uint8_t*>(p), [](uint8_t* q) { (void)hipFree(q); });
  return hipSuccess;
}
}  // namespace

struct qlinear_plan {
  ql_desc d;
  std::vector<int32_t> seg;  // host copy, n_segments + 1
  std::vector<int32_t> kseg; // input branch offsets, nks + 1 ({0, K} without branches)
  int nks = 1;
  int device = -1;
  // The GEMM (k_gemm1.hip) reads the stored codes and applies the TASQ
  // depth itself: every plan but the single-Hadamard one and those with 3
  // or 4 input branches. Views of such plans share the weights.
  bool depth_in_gemm = false;
  bool packed4 = false;      // 4-bit codes stored two per byte (depth_in_gemm plans)
  int w_lsb_k = 0;           // TASQ depth the GEMM applies (views of depth_in_gemm plans)
  DevBuf wq;                 // GEMM weights: codes int8 [N,K], packed 4-bit [N,K/2], or
                             // the two planes of H W_int^T, int8 [2 * roundup(N,16), K]
                             // (single Hadamard)
  DevBuf wint;               // single Hadamard: the codes W_int, int8 [N,K]
  DevBuf sw;                 // weight scales [nks, N] (float)
  float* ypart = nullptr;    // 3-4 input branches: the GEMM's partial-sum workspace
  ql::ReduceWs* ws = nullptr;
};

namespace {

thread_local std::string g_err;

ql_status fail(ql_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ql_status ok() {
  g_err.clear();
  return QL_OK;
}

ql_status hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? QL_ERR_OOM : QL_ERR_HIP, "%s: %s", what,
              hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int qmax(int bits) { return (1 << (bits - 1)) - 1; }

ql_status check_desc(const ql_desc* d) {
  if (!d) return fail(QL_ERR_ARG, "descriptor is NULL");
  if (d->N < 1) return fail(QL_ERR_ARG, "N = %d must be >= 1", d->N);
  if (d->K < 16 || d->K > 65536) return fail(QL_ERR_ARG, "K = %d must be in [16, 65536]", d->K);
  if ((d->w_bits != 4 && d->w_bits != 8) || (d->a_bits != 4 && d->a_bits != 8))
    return fail(QL_ERR_ARG, "w_bits = %d and a_bits = %d must each be 4 or 8", d->w_bits, d->a_bits);
  const bool any4 = d->w_bits == 4 || d->a_bits == 4;
  if (any4 && d->K % 32 != 0)
    return fail(QL_ERR_ARG, "K = %d must be a multiple of 32 with 4-bit codes", d->K);
  if (d->K % 16 != 0) return fail(QL_ERR_ARG, "K = %d must be a multiple of 16", d->K);
  const int hb = d->hadamard_block;
  if (hb != 0) {
    if (hb < 0 || (hb & (hb - 1)) != 0)
      return fail(QL_ERR_ARG, "hadamard_block = %d must be 0 or a power of two", hb);
    if (d->K % hb != 0)
      return fail(QL_ERR_ARG, "K = %d is not a multiple of hadamard_block = %d", d->K, hb);
    if (hb < 4 || hb > 128)
      return fail(QL_ERR_UNSUPPORTED, "hadamard_block = %d: supported blocks are 4..128", hb);
  }
  if (d->w_scale_mode != QL_WSCALE_PER_TENSOR && d->w_scale_mode != QL_WSCALE_PER_SEGMENT &&
      d->w_scale_mode != QL_WSCALE_PER_CHANNEL)
    return fail(QL_ERR_ARG, "bad w_scale_mode %d", (int)d->w_scale_mode);
  if (d->a_scale_mode != QL_ASCALE_DUAL && d->a_scale_mode != QL_ASCALE_SYMMETRIC)
    return fail(QL_ERR_ARG, "bad a_scale_mode %d", (int)d->a_scale_mode);
  if (d->x_dtype != QL_F32 && d->x_dtype != QL_BF16)
    return fail(QL_ERR_ARG, "bad x_dtype %d", (int)d->x_dtype);
  if (d->single_hadamard != 0 && d->single_hadamard != 1)
    return fail(QL_ERR_ARG, "single_hadamard = %d must be 0 or 1", d->single_hadamard);
  if (d->single_hadamard && hb == 0)
    return fail(QL_ERR_ARG, "single_hadamard needs hadamard_block > 0");
  if (d->single_hadamard && d->a_scale_mode != QL_ASCALE_SYMMETRIC)
    return fail(QL_ERR_UNSUPPORTED, "single_hadamard supports SYMMETRIC activation scales only");
  if (d->n_k_segments < 0)
    return fail(QL_ERR_ARG, "n_k_segments = %d must be >= 0", d->n_k_segments);
  if (d->n_k_segments > 1) {
    const int S = d->n_k_segments;
    if (S > ql::kMaxKSeg)
      return fail(QL_ERR_UNSUPPORTED, "n_k_segments = %d: at most %d input branches", S,
                  ql::kMaxKSeg);
    if (!d->k_seg_offsets) return fail(QL_ERR_ARG, "k_seg_offsets is NULL with n_k_segments = %d", S);
    const int32_t* o = d->k_seg_offsets;
    if (o[0] != 0 || o[S] != d->K)
      return fail(QL_ERR_ARG, "input branches must start at 0 and end at K = %d", d->K);
    for (int j = 0; j < S; ++j)
      if (o[j + 1] <= o[j]) return fail(QL_ERR_ARG, "input branch %d is empty or descending", j);
    for (int j = 1; j < S; ++j)
      if (o[j] % 128 != 0)
        return fail(QL_ERR_UNSUPPORTED, "input branch offset %d is not a multiple of 128", o[j]);
    if (d->single_hadamard)
      return fail(QL_ERR_UNSUPPORTED, "single_hadamard with input branches");
  }
  if (d->n_segments < 1) return fail(QL_ERR_ARG, "n_segments = %d must be >= 1", d->n_segments);
  if (d->n_segments > 1 && !d->seg_offsets)
    return fail(QL_ERR_ARG, "seg_offsets is NULL with n_segments = %d", d->n_segments);
  if (d->seg_offsets) {
    const int32_t* o = d->seg_offsets;
    if (o[0] != 0 || o[d->n_segments] != d->N)
      return fail(QL_ERR_ARG, "segments must start at 0 and end at N = %d", d->N);
    for (int g = 0; g < d->n_segments; ++g)
      if (o[g + 1] <= o[g]) return fail(QL_ERR_ARG, "segment %d is empty or descending", g);
  }
  return QL_OK;
}

// Partial-sum workspace of the single-Hadamard / many-branch GEMM for plans
// with 3 or 4 input branches (one block per compute unit of the device).
hipError_t alloc_ypart(struct qlinear_plan* p) {
  if (p->depth_in_gemm || p->nks <= 1) return hipSuccess;
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) return e;
  return hipMalloc(&p->ypart, ql::gemm_ypart_bytes(cus));
}

// Rows of the weight matrix the GEMM reads: N, or the hi/lo planes of every
// 16 output channels for the single Hadamard.
size_t gemm_weight_rows(const ql_desc& d) {
  return d.single_hadamard ? (size_t)2 * (((size_t)d.N + 15) / 16 * 16) : (size_t)d.N;
}

ql_status check_plan(qlinear_plan_t p) {
  if (!p) return fail(QL_ERR_ARG, "plan is NULL");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QL_ERR_HIP, "hipGetDevice failed");
  if (dev != p->device)
    return fail(QL_ERR_ARG, "current device %d is not the plan's device %d", dev, p->device);
  return QL_OK;
}

void free_plan(struct qlinear_plan* p) {
  if (!p) return;
  if (p->ypart) (void)hipFree(p->ypart);
  if (p->ws) (void)hipFree(p->ws);
  delete p;
}

// Two plans with the same descriptor and segments: weights of one can stand
// in for the other's in every call.
bool same_layer(const struct qlinear_plan* a, const struct qlinear_plan* b) {
  const ql_desc &x = a->d, &y = b->d;
  return x.N == y.N && x.K == y.K && x.w_bits == y.w_bits && x.a_bits == y.a_bits &&
         x.hadamard_block == y.hadamard_block && x.n_segments == y.n_segments &&
         x.w_scale_mode == y.w_scale_mode && x.a_scale_mode == y.a_scale_mode &&
         x.x_dtype == y.x_dtype && x.single_hadamard == y.single_hadamard && a->seg == b->seg &&
         a->kseg == b->kseg && a->device == b->device;
}

// Plans whose GEMM does not apply the depth (single Hadamard: the planes
// are built from the truncated codes; 3-4 input branches): enqueue view's
// weights = base's codes with k low magnitude bits cleared, and base's
// scales.
ql_status enqueue_lsb(struct qlinear_plan* view, const struct qlinear_plan* base, int k,
                      hipStream_t s) {
  const int64_t nbytes = (int64_t)base->d.N * base->d.K;
  const bool single = base->d.single_hadamard != 0;
  hipError_t e = ql::launch_truncate_weights(
      single ? base->wint.get() : base->wq.get(), nbytes, k,
      single ? view->wint.get() : view->wq.get(), reinterpret_cast<const float*>(base->sw.get()),
      reinterpret_cast<float*>(view->sw.get()), base->nks * base->d.N, s);
  if (e != hipSuccess) return hip_fail(e, "truncating weight codes");
  if (single) {  // rebuild the hi/lo planes from the truncated codes
    e = ql::launch_fwht_split(view->wint.get(), base->d.N, base->d.K, base->d.hadamard_block,
                              view->wq.get(), s);
    if (e != hipSuccess) return hip_fail(e, "single-Hadamard weight planes");
  }
  return QL_OK;
}

}  // namespace

// Reduction workspace of qlinear_quantize_act_noalloc: one copy per device,
// holding every partial maximum a call can write (kMaxKSeg branches x
// kMaxReduceBlocks pairs, 32 KiB) and the one-pass quantizer's exchange
// words (kMaxKSeg branches x 2 x kMaxReduceBlocks tagged 64-bit words,
// 64.25 KiB; zero when the library is loaded). Host code never passes `scratch`
// itself to a kernel (that name is a host-side stand-in): it passes the
// device address looked up once per device below.
static __device__ __align__(256) uint8_t scratch[sizeof(ql::ReduceWs)] = {};

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on device `dev` (the current device), looked
// up on the first call there and kept.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Sequence numbers of quantize calls, never 0 (the one-pass quantizer's
// barrier flags start at 0).
std::atomic<uint32_t> g_seq{0};
uint32_t next_seq() {
  uint32_t v = g_seq.fetch_add(1) + 1;
  while (v == 0) v = g_seq.fetch_add(1) + 1;
  return v;
}

// Shared body of qlinear_quantize_act and its no-allocation variant: `ws`
// receives the per-block partial maxima of a dynamic-scale call.
ql_status quantize_impl(qlinear_plan_t p, const void* X, int32_t M, int32_t lsb_k,
                        const float* static_scales, void* codes, float* act_scales,
                        ql::ReduceWs* ws, void* stream) {
  if (M < 0) return fail(QL_ERR_ARG, "M = %d must be >= 0", M);
  if (lsb_k < 0 || lsb_k >= p->d.a_bits)
    return fail(QL_ERR_ARG, "lsb_k = %d must be in [0, %d)", lsb_k, p->d.a_bits);
  if (M == 0) return ok();  // empty tensors may carry NULL data pointers
  if (!X || !codes || !act_scales) return fail(QL_ERR_ARG, "X, codes or act_scales is NULL");
  const bool bf16 = p->d.x_dtype == QL_BF16;
  if (!aligned(X, bf16 ? 8 : 16)) return fail(QL_ERR_ARG, "X is not %d-byte aligned", bf16 ? 8 : 16);
  if (!aligned(codes, 16)) return fail(QL_ERR_ARG, "codes must be 16-byte aligned");
  if (!aligned(act_scales, 4) || (static_scales && !aligned(static_scales, 4)))
    return fail(QL_ERR_ARG, "scale pointers must be 4-byte aligned");
  ql::QuantArgs a;
  a.X = X;
  a.nunits = (int64_t)M * p->d.K / 4;
  a.codes = codes;
  a.act_scales = act_scales;
  a.static_scales = static_scales;
  a.ws = ws;
  a.reduce_blocks = 0;
  a.qa = (float)qmax(p->d.a_bits);
  a.keep_mask = ~((1 << lsb_k) - 1);
  a.sym = p->d.a_scale_mode == QL_ASCALE_SYMMETRIC;
  a.nks = p->nks;
  a.k_units = p->d.K / 4;
  for (int j = 0; j < ql::kMaxKSeg; ++j) a.ks_units[j] = j < p->nks ? p->kseg[j] / 4 : a.k_units;
  a.seq = next_seq();
  hipError_t e = ql::launch_quantize(a, bf16, p->d.hadamard_block, p->d.a_bits == 4,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching quantize");
  return ok();
}

}  // namespace

namespace ql {
// Status reporting for the host-only entry points in other files.
ql_status set_error(ql_status st, const char* msg) {
  if (st == QL_OK) return ok();
  return fail(st, "%s", msg);
}
}  // namespace ql

extern "C" {

const char* qlinear_last_error(void) { return g_err.c_str(); }

const char* qlinear_version(void) { return "qlinear 0.1.0 gfx950"; }

ql_status qlinear_plan(const ql_desc* d, const float* W, void* stream, qlinear_plan_t* out) {
  ql_status st = check_desc(d);
  if (st != QL_OK) return st;
  if (!W || !out) return fail(QL_ERR_ARG, "W or out is NULL");
  if (!aligned(W, 16)) return fail(QL_ERR_ARG, "W must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto* p = new struct qlinear_plan();
  p->d = *d;
  if (d->seg_offsets) {
    p->seg.assign(d->seg_offsets, d->seg_offsets + d->n_segments + 1);
  } else {
    p->seg = {0, d->N};
    p->d.n_segments = 1;
  }
  p->d.seg_offsets = nullptr;
  if (d->n_k_segments > 1) {
    p->kseg.assign(d->k_seg_offsets, d->k_seg_offsets + d->n_k_segments + 1);
  } else {
    p->kseg = {0, d->K};
    p->d.n_k_segments = 1;
  }
  p->nks = (int)p->kseg.size() - 1;
  p->d.k_seg_offsets = nullptr;
  if (hipGetDevice(&p->device) != hipSuccess) {
    free_plan(p);
    return fail(QL_ERR_HIP, "hipGetDevice failed");
  }
  const int64_t N = d->N, K = d->K;
  // 4-bit codes are stored two per byte [N, K/2] where the GEMM unpacks
  // them (depth_in_gemm plans), one per byte otherwise.
  const bool single = d->single_hadamard != 0;
  p->depth_in_gemm = !single && p->nks <= 2;
  p->packed4 = p->depth_in_gemm && d->w_bits == 4;
  const size_t wbytes = (size_t)(N * K);
  const size_t gbytes = single ? gemm_weight_rows(*d) * (size_t)K : p->packed4 ? wbytes / 2 : wbytes;
  float* rot = nullptr;
  uint32_t* rowmax = nullptr;
  int32_t* segd = nullptr;
  uint8_t* codes8 = nullptr;  // packed plans: the codes one per byte, before packing
  hipError_t e = hipSuccess;
  auto cleanup = [&]() {
    if (rot) (void)hipFree(rot);
    if (rowmax) (void)hipFree(rowmax);
    if (segd) (void)hipFree(segd);
    if (codes8) (void)hipFree(codes8);
  };
  // On failure, let the work already enqueued finish before its buffers go.
#define QL_TRY(expr, what)                \
  do {                                    \
    e = (expr);                           \
    if (e != hipSuccess) {                \
      (void)hipStreamSynchronize(s);      \
      cleanup();                          \
      free_plan(p);                       \
      return hip_fail(e, what);           \
    }                                     \
  } while (0)
  QL_TRY(dev_alloc(p->wq, gbytes), "allocating weight codes");
  if (single) QL_TRY(dev_alloc(p->wint, wbytes), "allocating unrotated weight codes");
  if (p->packed4) QL_TRY(hipMalloc(&codes8, wbytes), "allocating unpacked weight codes");
  QL_TRY(dev_alloc(p->sw, (size_t)p->nks * N * sizeof(float)), "allocating weight scales");
  QL_TRY(hipMalloc(&p->ws, sizeof(ql::ReduceWs)), "allocating reduction workspace");
  QL_TRY(hipMemsetAsync(p->ws, 0, sizeof(ql::ReduceWs), s), "clearing reduction workspace");
  QL_TRY(hipMalloc(&rowmax, N * sizeof(uint32_t)), "allocating row maxima");
  QL_TRY(alloc_ypart(p), "allocating partial-sum workspace");
  // Offsets that define the scale groups: the given segments for
  // PER_SEGMENT, one group [0,N) for PER_TENSOR (unused for PER_CHANNEL).
  const int mode = d->w_scale_mode == QL_WSCALE_PER_SEGMENT  ? 1
                   : d->w_scale_mode == QL_WSCALE_PER_TENSOR ? 0
                                                             : 2;
  const std::vector<int32_t> groups =
      mode == 1 ? p->seg : std::vector<int32_t>{0, (int32_t)N};
  const int ngroups = (int)groups.size() - 1;
  QL_TRY(hipMalloc(&segd, groups.size() * sizeof(int32_t)), "allocating segment offsets");
  QL_TRY(hipMemcpyAsync(segd, groups.data(), groups.size() * sizeof(int32_t),
                        hipMemcpyHostToDevice, s),
         "copying segment offsets");
  const float* src = W;
  if (d->hadamard_block && !single) {
    QL_TRY(hipMalloc(&rot, N * K * sizeof(float)), "allocating rotation buffer");
    QL_TRY(hipMemcpyAsync(rot, W, N * K * sizeof(float), hipMemcpyDeviceToDevice, s),
           "copying W");
    QL_TRY(ql::launch_rotate_rows(rot, N * K / 4, d->hadamard_block, s), "rotating W");
    src = rot;
  }
  const float qw = (float)qmax(d->w_bits);
  // Every input branch (the whole row without branches) has its own scales
  // over its own columns.
  uint8_t* codes_out = single ? p->wint.get() : p->packed4 ? codes8 : p->wq.get();
  for (int j = 0; j < p->nks; ++j) {
    const int c0 = p->kseg[j], cw = p->kseg[j + 1] - p->kseg[j];
    float* swj = reinterpret_cast<float*>(p->sw.get()) + (int64_t)j * N;
    QL_TRY(ql::launch_row_absmax(src, (int)N, (int)K, c0, cw, rowmax, s), "weight row maxima");
    QL_TRY(ql::launch_weight_scales(rowmax, (int)N, mode, segd, ngroups, qw, swj, s),
           "weight scales");
    QL_TRY(ql::launch_quantize_weights(src, swj, (int)N, (int)K, c0, cw, qw, codes_out, s),
           "weight codes");
  }
  if (p->packed4) QL_TRY(ql::launch_pack4(codes8, N * K, p->wq.get(), s), "packing weight codes");
  if (single) {
    QL_TRY(hipMemsetAsync(p->wq.get(), 0, gbytes, s), "clearing weight planes");
    QL_TRY(ql::launch_fwht_split(p->wint.get(), (int)N, (int)K, d->hadamard_block, p->wq.get(), s),
           "single-Hadamard weight planes");
  }
  QL_TRY(hipStreamSynchronize(s), "synchronising plan stream");
#undef QL_TRY
  cleanup();
  *out = p;
  return ok();
}

ql_status qlinear_plan_destroy(qlinear_plan_t p) {
  free_plan(p);
  return ok();
}

ql_status qlinear_plan_lsb_view(qlinear_plan_t base, int32_t w_lsb_k, void* stream,
                                qlinear_plan_t* out) {
  ql_status st = check_plan(base);
  if (st != QL_OK) return st;
  if (!out) return fail(QL_ERR_ARG, "out is NULL");
  if (w_lsb_k < 0 || w_lsb_k >= base->d.w_bits)
    return fail(QL_ERR_ARG, "w_lsb_k = %d must be in [0, %d)", w_lsb_k, base->d.w_bits);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto* v = new struct qlinear_plan();
  v->d = base->d;
  v->seg = base->seg;
  v->kseg = base->kseg;
  v->nks = base->nks;
  v->device = base->device;
  v->depth_in_gemm = base->depth_in_gemm;
  v->packed4 = base->packed4;
  if (base->depth_in_gemm) {
    // TASQ's one stored buffer: the view shares the base's codes and scales
    // and carries the depth, which the GEMM applies as it loads the codes
    // (clearing k bits after k' cleared clears max(k, k')).
    v->wq = base->wq;
    v->sw = base->sw;
    v->w_lsb_k = w_lsb_k > base->w_lsb_k ? w_lsb_k : base->w_lsb_k;
    hipError_t e = hipMalloc(&v->ws, sizeof(ql::ReduceWs));
    if (e == hipSuccess) e = hipMemsetAsync(v->ws, 0, sizeof(ql::ReduceWs), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      free_plan(v);
      return hip_fail(e, "allocating view plan");
    }
    *out = v;
    return ok();
  }
  const size_t wbytes = (size_t)base->d.N * base->d.K;
  const size_t gbytes = gemm_weight_rows(base->d) * (size_t)base->d.K;
  hipError_t e = dev_alloc(v->wq, gbytes);
  if (e == hipSuccess) e = dev_alloc(v->sw, (size_t)base->nks * base->d.N * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&v->ws, sizeof(ql::ReduceWs));
  if (e == hipSuccess) e = hipMemsetAsync(v->ws, 0, sizeof(ql::ReduceWs), s);
  if (e == hipSuccess) e = alloc_ypart(v);
  if (e == hipSuccess && base->d.single_hadamard) {
    e = dev_alloc(v->wint, wbytes);
    // rows past N of the planes stay zero for the life of the view
    if (e == hipSuccess) e = hipMemsetAsync(v->wq.get(), 0, gbytes, s);
  }
  if (e != hipSuccess) {
    free_plan(v);
    return hip_fail(e, "allocating view plan");
  }
  st = enqueue_lsb(v, base, w_lsb_k, s);
  if (st != QL_OK) {
    (void)hipStreamSynchronize(s);
    free_plan(v);
    return st;
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_plan(v);
    return hip_fail(e, "synchronising view stream");
  }
  *out = v;
  return ok();
}

ql_status qlinear_plan_lsb_update(qlinear_plan_t view, qlinear_plan_t base, int32_t w_lsb_k,
                                  void* stream) {
  ql_status st = check_plan(base);
  if (st != QL_OK) return st;
  st = check_plan(view);
  if (st != QL_OK) return st;
  if (view == base) return fail(QL_ERR_ARG, "view and base are the same plan");
  if (!same_layer(view, base))
    return fail(QL_ERR_ARG, "view and base differ in descriptor or segments");
  if (w_lsb_k < 0 || w_lsb_k >= base->d.w_bits)
    return fail(QL_ERR_ARG, "w_lsb_k = %d must be in [0, %d)", w_lsb_k, base->d.w_bits);
  if (view->depth_in_gemm) {  // a new depth over the base's buffer, no data moved
    view->wq = base->wq;
    view->sw = base->sw;
    view->w_lsb_k = w_lsb_k > base->w_lsb_k ? w_lsb_k : base->w_lsb_k;
    return ok();
  }
  st = enqueue_lsb(view, base, w_lsb_k, reinterpret_cast<hipStream_t>(stream));
  if (st != QL_OK) return st;
  return ok();
}

ql_status qlinear_plan_weights(qlinear_plan_t p, int8_t* w_codes, float* w_scales, void* stream) {
  ql_status st = check_plan(p);
  if (st != QL_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (w_codes) {
    const int64_t n = (int64_t)p->d.N * p->d.K;
    uint8_t* out = reinterpret_cast<uint8_t*>(w_codes);
    if (p->packed4) {
      e = ql::launch_unpack4(p->wq.get(), n, p->w_lsb_k, out, s);
    } else if (p->w_lsb_k > 0) {
      if (!aligned(w_codes, 16)) return fail(QL_ERR_ARG, "w_codes must be 16-byte aligned");
      e = ql::launch_truncate_weights(p->wq.get(), n, p->w_lsb_k, out, nullptr, nullptr, 0, s);
    } else {
      e = hipMemcpyAsync(w_codes, p->d.single_hadamard ? p->wint.get() : p->wq.get(), (size_t)n,
                         hipMemcpyDeviceToDevice, s);
    }
    if (e != hipSuccess) return hip_fail(e, "copying weight codes");
  }
  if (w_scales) {
    e = hipMemcpyAsync(w_scales, p->sw.get(), (size_t)p->nks * p->d.N * sizeof(float),
                       hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "copying weight scales");
  }
  return ok();
}

ql_status qlinear_quantize_act(qlinear_plan_t p, const void* X, int32_t M, int32_t lsb_k,
                               const float* static_scales, void* codes, float* act_scales,
                               void* stream) {
  ql_status st = check_plan(p);
  if (st != QL_OK) return st;
  return quantize_impl(p, X, M, lsb_k, static_scales, codes, act_scales, p->ws, stream);
}

ql_status qlinear_quantize_act_noalloc(qlinear_plan_t p, const void* X, int32_t M,
                                       int32_t lsb_k, const float* static_scales, void* codes,
                                       float* act_scales, void* stream) {
  ql_status st = check_plan(p);
  if (st != QL_OK) return st;
  // The scratch holds kMaxKSeg branches of kMaxReduceBlocks partial pairs;
  // the reduce grid never exceeds kMaxReduceBlocks blocks, whatever M.
  if (p->nks > ql::kMaxKSeg)
    return fail(QL_ERR_UNSUPPORTED, "%d input branches exceed the scratch's %d", p->nks,
                ql::kMaxKSeg);
  void* ws = nullptr;
  const hipError_t e = scratch_address(p->device, &ws);
  if (e != hipSuccess) return hip_fail(e, "looking up the reduction scratch");
  return quantize_impl(p, X, M, lsb_k, static_scales, codes, act_scales,
                       reinterpret_cast<ql::ReduceWs*>(ws), stream);
}

ql_status qlinear_gemm(qlinear_plan_t p, const void* codes, const float* act_scales, int32_t M,
                       int32_t cfg, float w, float* Y, int32_t* acc_dbg, void* stream) {
  ql_status st = check_plan(p);
  if (st != QL_OK) return st;
  if (M < 0) return fail(QL_ERR_ARG, "M = %d must be >= 0", M);
  if (M > (1 << 23)) return fail(QL_ERR_UNSUPPORTED, "M = %d exceeds 8388608 rows", M);
  if (cfg != 0 && cfg != 1) return fail(QL_ERR_ARG, "cfg = %d must be 0 or 1", cfg);
  if (cfg && (M % 2)) return fail(QL_ERR_ARG, "M = %d must be even with cfg = 1", M);
  if (M == 0) return ok();  // empty tensors may carry NULL data pointers
  if (!codes || !act_scales || !Y) return fail(QL_ERR_ARG, "codes, act_scales or Y is NULL");
  if (!aligned(codes, 16)) return fail(QL_ERR_ARG, "codes must be 16-byte aligned");
  if (!aligned(Y, 4) || !aligned(act_scales, 4) || (acc_dbg && !aligned(acc_dbg, 4)))
    return fail(QL_ERR_ARG, "Y, act_scales and acc_dbg must be 4-byte aligned");
  ql::GemmArgs g;
  g.A = reinterpret_cast<const uint8_t*>(codes);
  g.W = p->wq.get();
  g.act_scales = act_scales;
  g.w_scales = reinterpret_cast<const float*>(p->sw.get());
  g.Y = Y;
  g.dbg = acc_dbg;
  g.M = M;
  g.N = (int)gemm_weight_rows(p->d);
  g.Nout = p->d.N;
  g.K = p->d.K;
  g.Mh = cfg ? M / 2 : M;
  g.lda = p->d.a_bits == 4 ? p->d.K / 2 : p->d.K;
  g.ldw = p->packed4 ? p->d.K / 2 : p->d.K;
  if ((int64_t)M * g.lda >= ((int64_t)1 << 31) || (int64_t)g.N * g.ldw >= ((int64_t)1 << 31))
    return fail(QL_ERR_UNSUPPORTED, "codes or weights of 2 GiB or more (M = %d)", M);
  // Output offsets within a 128-row tile are 32-bit byte offsets.
  if ((int64_t)g.N * 4 * 128 >= ((int64_t)1 << 31))
    return fail(QL_ERR_UNSUPPORTED, "N = %d: a 128-row block of Y reaches 2 GiB", g.N);
  g.guidance = w;
  g.inv_b = p->d.hadamard_block ? 1.0f / (float)p->d.hadamard_block : 1.0f;
  g.nks = p->nks;
  g.ypart_ws = p->ypart;
  for (int j = 0; j < ql::kMaxKSeg; ++j)
    g.ks_end[j] = j + 1 < p->nks ? p->kseg[j + 1] / 128 : 0x7FFFFFFF;
  for (int j = 0; j <= ql::kMaxKSeg; ++j) g.kofs[j] = j < p->nks ? p->kseg[j] : p->d.K;
  for (int j = 0; j < ql::kMaxKSeg; ++j) {
    const int steps = j < p->nks ? (p->kseg[j + 1] - p->kseg[j] + 127) / 128 : 0;
    g.ksteps[j] = (steps + 2) / 3 * 3;
  }
  // Plans that keep a truncated copy hand the GEMM depth 0 (the copy is
  // already truncated).
  g.w_lsb_k = p->depth_in_gemm ? p->w_lsb_k : 0;
  const int a4 = p->d.a_bits == 4, sym = p->d.a_scale_mode == QL_ASCALE_SYMMETRIC;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Kernel choice: k_gemm.hip for single-Hadamard and 3-4-branch plans, and
  // for int8 W8A8 DualScale CFG layers with 144-column tiles and no rotation,
  // at any TASQ depth (measured faster there); k_gemm1.hip for everything
  // else.
  const bool plain_w8a8_cfg = p->depth_in_gemm && !p->packed4 && p->nks == 1 && !a4 && !sym &&
                              cfg && g.N % 144 == 0 && p->d.hadamard_block == 0;
  const hipError_t e = p->depth_in_gemm && !plain_w8a8_cfg
                           ? ql::launch_gemm1(g, a4, sym, cfg, p->packed4, s)
                           : ql::launch_gemm(g, a4, sym, cfg, p->d.single_hadamard, s);
  if (e != hipSuccess) return hip_fail(e, "launching gemm");
  return ok();
}

ql_status qlinear_probe_mfma(const void* operands, int32_t iters, int32_t waves_per_simd,
                             int32_t* sink, int64_t sink_len, void* stream) {
  if (!operands || !sink) return fail(QL_ERR_ARG, "operands or sink is NULL");
  if (iters < 0 || iters > (1 << 24)) return fail(QL_ERR_ARG, "iters = %d must be in [0, 2^24]", iters);
  if (waves_per_simd != 1 && waves_per_simd != 2)
    return fail(QL_ERR_ARG, "waves_per_simd = %d must be 1 or 2", waves_per_simd);
  if (!aligned(operands, 16) || !aligned(sink, 4))
    return fail(QL_ERR_ARG, "operands must be 16-byte and sink 4-byte aligned");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "querying the compute units");
  const int64_t need = (int64_t)cus * 256 * waves_per_simd;
  if (sink_len < need)
    return fail(QL_ERR_ARG, "sink holds %lld int32, the grid writes %lld", (long long)sink_len,
                (long long)need);
  e = ql::launch_probe_mfma(operands, iters, waves_per_simd, cus, sink,
                            reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching the MFMA probe");
  return ok();
}

ql_status qlinear_cfg_combine(const float* Y, int32_t M, int32_t N, float w, float* out,
                              void* stream) {
  if (M < 0 || N < 1) return fail(QL_ERR_ARG, "M = %d, N = %d: need M >= 0, N >= 1", M, N);
  if (M % 2) return fail(QL_ERR_ARG, "M = %d must be even", M);
  if (M == 0) return ok();
  if (!Y || !out) return fail(QL_ERR_ARG, "Y or out is NULL");
  if (!aligned(Y, 4) || !aligned(out, 4)) return fail(QL_ERR_ARG, "Y and out must be 4-byte aligned");
  const int64_t half = (int64_t)(M / 2) * N;
  const uintptr_t y0 = reinterpret_cast<uintptr_t>(Y), y1 = y0 + 2 * half * sizeof(float);
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + half * sizeof(float);
  if (half > 0 && o0 < y1 && y0 < o1) return fail(QL_ERR_ARG, "out overlaps Y");
  if (half == 0) return ok();
  hipError_t e = ql::launch_cfg_combine(Y, half, w, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "launching cfg_combine");
  return ok();
}

}  // extern "C"
