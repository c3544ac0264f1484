// C ABI of the library (include/moe.h): argument validation, workspace layout
// and the launch sequence.  Every check that needs no device runs first, so a
// bad call is refused before the HIP runtime is touched; then the device checks
// (gfx950, pointers on the stream's device); then the kernels are enqueued.
//
// The refusals mirror the pages' guards, which all fire before any kernel work:
// non-bf16 hidden states (ValueError), non-int8 FP4 weights
// (NotImplementedError), a model spread over several devices in one process
// (RuntimeError), and a device that cannot serve the dtypes ("DeepGEMM
// experts selected on a model spanning multiple CUDA devices", the record's
// source; "DeepGEMM Mega MoE requires FP4-packed expert weights (dtype=int8)",
// section "Source").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <utility>
#include <string>
#include <vector>

#include "internal.h"
#include "moe.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_fmt(int f) { return f == MOE_FMT_FP8_B128 || f == MOE_FMT_MXFP8A_MXFP4W || f == MOE_FMT_BF16; }

constexpr int kMaxE = 512;
constexpr int kMaxK = 64;
constexpr int kMaxClockStamps = 4096;

// ------------------------------------------------------------ device checks
struct DeviceInfo {
  bool probed = false;
  bool gfx950 = false;
  int num_cus = 0;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

moe_status stream_device(hipStream_t stream, int* dev) {
  hipError_t e = hipStreamGetDevice(stream, dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status check_device(hipStream_t stream, int* dev_out, int* num_cus) {
  int dev = 0;
  moe_status st = stream_device(stream, &dev);
  if (st != MOE_OK) return st;
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.probed = true;
    if (!d.gfx950) {
      d.probed = false;
      return fail(MOE_ERR_ARCH, "device %d is %s; these kernels are built for gfx950 (MI355X)", dev,
                  prop.gcnArchName);
    }
  }
  *dev_out = dev;
  *num_cus = d.num_cus;
  return MOE_OK;
}

// A pointer must be device memory of `dev` (or host-registered memory mapped on it).
moe_status check_ptr(const void* p, int dev, const char* name) {
  if (!p) return MOE_OK;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "%s is not memory known to the HIP runtime", name);
  }
  if (attr.type == hipMemoryTypeDevice && attr.device != dev)
    return fail(MOE_ERR_DEVICE, "%s lives on device %d but the stream is on device %d (one device per process)", name,
                attr.device, dev);
  return MOE_OK;
}

// Every non-NULL pointer of the list must pass check_ptr.
moe_status check_ptrs(int dev, std::initializer_list<std::pair<const void*, const char*>> ptrs) {
  for (const auto& pr : ptrs) {
    const moe_status st = check_ptr(pr.first, dev, pr.second);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------- forward workspace
struct FwdLayout {
  size_t sorted_slot, offsets, act_codes, act_scales, h_codes, h_scales, slot_out, sort_ws, sched;
  // with the multi-workgroup sort (quantized formats): the activation scales
  // by sorted row, which the gate_up GEMM reads contiguously
  bool sorted_scales;
  size_t act_scales_sorted, total;
};

FwdLayout fwd_layout(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I, int fmt) {
  const size_t S = (size_t)T * k;
  const size_t A = 256;
  const bool mx = fmt == MOE_FMT_MXFP8A_MXFP4W;
  const bool bf = fmt == MOE_FMT_BF16;  // activations used as they are; h kept in bf16
  FwdLayout L;
  size_t o = 0;
  L.sorted_slot = o; o = align_up(o + 4 * S, A);
  L.offsets = o; o = align_up(o + 4 * (size_t)(E + 1), A);
  L.act_codes = o; o = align_up(o + (bf ? 0 : (size_t)T * H), A);
  L.act_scales = o; o = align_up(o + (bf ? 0 : mx ? (size_t)T * (H / 32) : 4 * (size_t)T * (H / 128)), A);
  L.h_codes = o; o = align_up(o + S * I * (bf ? 2 : 1), A);
  L.h_scales = o; o = align_up(o + (bf ? 0 : mx ? S * (I / 32) : 4 * S * (I / 128)), A);
  L.slot_out = o; o = align_up(o + 2 * S * H, A);
  L.sort_ws = o; o = align_up(o + moe::route_sort_ws_bytes((int32_t)S, E), A);
  L.sched = o; o = align_up(o + 2 * MOE_TILE_COUNTERS_BYTES, A);  // gate_up's and down's tile counters
  L.sorted_scales = !bf && moe::route_sort_multiblock((int32_t)S);
  L.act_scales_sorted = o;
  o = align_up(o + (!L.sorted_scales ? 0 : mx ? S * (H / 32) : 4 * S * (H / 128)), A);
  L.total = o;
  return L;
}

moe_status validate_weights(const moe_weights* w) {
  if (!w) return fail(MOE_ERR_NULL, "weights descriptor is NULL");
  if (!valid_fmt(w->fmt)) return fail(MOE_ERR_UNSUPPORTED, "unknown weight format %d", (int)w->fmt);
  if (w->E < 1 || w->E > kMaxE) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", w->E, kMaxE);
  if (w->H <= 0 || w->I <= 0 || w->H % 128 || w->I % 128)
    return fail(MOE_ERR_SHAPE, "H=%d and I=%d must be positive multiples of 128", w->H, w->I);
  if ((int64_t)2 * w->I * w->H >= (int64_t)1 << 31 || (int64_t)w->H * w->I >= (int64_t)1 << 31)
    return fail(MOE_ERR_SHAPE, "one expert's weight must stay below 2^31 elements");
  if (!w->w13 || !w->w2) return fail(MOE_ERR_NULL, "weight pointer is NULL");
  if (w->fmt != MOE_FMT_BF16 && (!w->w13_scale || !w->w2_scale)) return fail(MOE_ERR_NULL, "weight scale is NULL");
  return MOE_OK;
}

moe_status validate_gemm(const moe_gemm_args* a) {
  if (!a) return fail(MOE_ERR_NULL, "gemm args are NULL");
  moe_status st = validate_weights(a->weights);
  if (st != MOE_OK) return st;
  if (a->which != 0 && a->which != 1) return fail(MOE_ERR_UNSUPPORTED, "which=%d is neither 0 (gate_up) nor 1 (down)", a->which);
  if (a->max_rows < 0) return fail(MOE_ERR_SHAPE, "max_rows=%d", a->max_rows);
  if (a->a_rows < 0 || (int64_t)a->a_rows * 128 >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "a_rows=%d", a->a_rows);
  if (!a->a_row_index && a->a_rows < a->max_rows)
    return fail(MOE_ERR_SHAPE, "without a row index A needs max_rows=%d rows, has %d", a->max_rows, a->a_rows);
  if (a->a_row_index && a->a_row_divisor < 1) return fail(MOE_ERR_SHAPE, "a_row_divisor must be >= 1");
  if (!a->a_codes || !a->expert_offsets || (a->weights->fmt != MOE_FMT_BF16 && !a->a_scales))
    return fail(MOE_ERR_NULL, "an operand pointer is NULL");
  if (a->weights->fmt == MOE_FMT_BF16 &&
      (int64_t)a->a_rows * (a->which == 0 ? a->weights->H : a->weights->I) * 2 >= (int64_t)1 << 32)
    return fail(MOE_ERR_SHAPE, "the bf16 A operand must stay below 4 GiB");
  switch (a->epilogue) {
    case MOE_EPI_STORE_F32:
      if (!a->c_f32) return fail(MOE_ERR_NULL, "c_f32 is NULL");
      break;
    case MOE_EPI_SWIGLU_QUANT:
      if (a->which != 0) return fail(MOE_ERR_UNSUPPORTED, "the SwiGLU epilogue runs on the gate_up weight (which = 0)");
      if (!a->h_codes || (a->weights->fmt != MOE_FMT_BF16 && !a->h_scales))
        return fail(MOE_ERR_NULL, "h_codes / h_scales are NULL");
      if (a->has_swiglu_limit && !(std::isfinite(a->swiglu_limit) && a->swiglu_limit > 0.0f))
        return fail(MOE_ERR_SHAPE, "swiglu_limit must be finite and > 0");
      break;
    case MOE_EPI_WEIGHTED_SCATTER:
      if (!a->slot_out || !a->top_k_weights || !a->slot_of_row)
        return fail(MOE_ERR_NULL, "slot_out / top_k_weights / slot_of_row are NULL");
      break;
    default:
      return fail(MOE_ERR_UNSUPPORTED, "unknown epilogue %d", (int)a->epilogue);
  }
  if ((uintptr_t)a->tile_counters % 8)
    return fail(MOE_ERR_SHAPE, "tile_counters must be 8-byte aligned (64-bit counters)");
  // the epilogue's outputs must not alias what the launch reads
  const void* outs[] = {a->epilogue == MOE_EPI_STORE_F32 ? (const void*)a->c_f32 : nullptr,
                        a->epilogue == MOE_EPI_SWIGLU_QUANT ? (const void*)a->h_codes : nullptr,
                        a->epilogue == MOE_EPI_SWIGLU_QUANT ? (const void*)a->h_scales : nullptr,
                        a->epilogue == MOE_EPI_WEIGHTED_SCATTER ? (const void*)a->slot_out : nullptr};
  const void* ins[] = {a->a_codes, a->a_scales, a->a_row_index, a->expert_offsets, a->a_scales_sorted,
                       a->top_k_weights, a->slot_of_row, a->tile_counters};
  for (const void* o : outs)
    for (const void* i : ins)
      if (o && o == i) return fail(MOE_ERR_UNSUPPORTED, "an epilogue output aliases an input of the launch");
  return MOE_OK;
}

moe::GemmParams to_params(const moe_gemm_args* a) {
  const moe_weights* w = a->weights;
  moe::GemmParams p{};
  p.a_codes = a->a_codes;
  p.a_scales = a->a_scales;
  p.a_row_index = a->a_row_index;
  p.a_row_div = a->a_row_index ? a->a_row_divisor : 1;
  p.a_rows = a->a_rows;
  p.offsets = a->expert_offsets;
  p.E = w->E;
  p.b_codes = a->which == 0 ? w->w13 : w->w2;
  p.b_scales = a->which == 0 ? w->w13_scale : w->w2_scale;
  p.N = a->which == 0 ? 2 * w->I : w->H;
  p.K = a->which == 0 ? w->H : w->I;
  p.max_rows = a->max_rows;
  p.a_scales_sorted = w->fmt == MOE_FMT_BF16 ? nullptr : a->a_scales_sorted;
  p.c_f32 = a->c_f32;
  p.sched = a->tile_counters;
  p.h_codes = a->h_codes;
  p.h_scales = a->h_scales;
  p.has_limit = a->has_swiglu_limit ? 1 : 0;
  p.limit = a->swiglu_limit;
  p.slot_out = a->slot_out;
  p.top_k_weights = a->top_k_weights;
  p.slot_of_row = a->slot_of_row;
  return p;
}

// At most this many rows per expert on average (decode batches): the FP8 GEMM
// streams the weights through registers instead of LDS tiles.  Forward times
// (uniform routing) of the register-streaming against the tiled kernel: on the
// Qwen3-MoE shape 124 against 153 us at 10 rows, 131 against 156 at 12, 135
// against 156 at 14, 154 against 157 at 16; on the DeepSeek-V3 shape 1.85
// against 1.97 ms at 10 rows, 1.99 against 2.00 at 12, but 2.24 against 2.01
// at 14 and 2.66 against 2.03 at 16 (past 16 rows an expert needs a second
// 16-row tile, whose weights stream again).
constexpr int64_t kSkinnyRowsPerExpert = 12;

hipError_t launch_gemm(const moe::GemmParams& p, int fmt, int epi, bool paired, int num_cus, hipStream_t stream) {
  if (fmt == MOE_FMT_BF16) return moe::launch_gemm_bf16(p, epi, paired, num_cus, stream);
  if (fmt == MOE_FMT_FP8_B128) {
    if ((int64_t)p.max_rows <= kSkinnyRowsPerExpert * p.E)
      return moe::launch_gemm_fp8_skinny(p, epi, paired, num_cus, stream);
    return moe::launch_gemm_fp8_b128(p, epi, paired, num_cus, stream);
  }
  return moe::launch_gemm_mx(p, epi, paired, num_cus, stream);
}

// The forward behind both entry points; with a router, top_k_index and
// top_k_weights are outputs that the router fills before the sort reads them.
// The scratch of moe_experts_forward_noalloc: one array per GPU, in device
// memory for the life of the process.  Host code never uses its name as an
// address (on the host it is only a stand-in): its device address, per device,
// comes from hipGetSymbolAddress with that device current.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of `scratch` on device dev (looked up once per device).
moe_status scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MOE_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// ws_is_scratch: ws is the library's own scratch array (whose address the
// runtime's pointer query need not know), so it is not checked as a caller
// pointer.
moe_status forward_impl(const moe_weights* w, const uint16_t* hidden_states, const moe::RouterArgs* router,
                        const int32_t* top_k_index, const float* top_k_weights, int32_t T, int32_t k,
                        const moe_options* opt, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream,
                        bool ws_is_scratch = false) {
  moe_status st = validate_weights(w);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d < 0", T);
  if (k < 1 || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, %d]", k, kMaxK);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must stay below 2^31");
  if (opt && opt->expert_begin < 0) return fail(MOE_ERR_SHAPE, "expert_begin=%d < 0", opt->expert_begin);
  const bool has_limit = opt && opt->has_swiglu_limit;
  if (has_limit && !(std::isfinite(opt->swiglu_limit) && opt->swiglu_limit > 0.0f))
    return fail(MOE_ERR_SHAPE, "swiglu_limit must be finite and > 0");
  const bool stat = opt && opt->static_activation_scales;
  if (stat) {
    if (w->fmt == MOE_FMT_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "static activation scales need a quantized format (the bf16 experts quantize nothing)");
    const int32_t nb = w->H / (w->fmt == MOE_FMT_FP8_B128 ? 128 : 32);
    if (opt->act_scales_row_stride < 0 || (opt->act_scales_row_stride > 0 && opt->act_scales_row_stride < nb))
      return fail(MOE_ERR_SHAPE, "act_scales_row_stride=%d: 0 or at least one row of %d block scales",
                  opt->act_scales_row_stride, nb);
  }
  if (router) {
    if (router->n_experts < 1 || router->n_experts > kMaxE)
      return fail(MOE_ERR_SHAPE, "n_experts=%d outside [1, %d]", router->n_experts, kMaxE);
    if (k > router->n_experts) return fail(MOE_ERR_SHAPE, "k=%d exceeds n_experts=%d", k, router->n_experts);
  }
  if (w->fmt != MOE_FMT_BF16 && (int64_t)T * k * 128 >= (int64_t)1 << 31)
    return fail(MOE_ERR_SHAPE, "T*k*128 must stay below 2^31 (32-bit row offsets in a K plane)");
  if (w->fmt == MOE_FMT_BF16 && ((int64_t)T * w->H * 2 >= (int64_t)1 << 32 ||
                                 (int64_t)T * k * w->I * 2 >= (int64_t)1 << 32))
    return fail(MOE_ERR_SHAPE, "bf16 experts: hidden_states and h must each stay below 4 GiB");
  if (T == 0) return ok();
  if (!hidden_states || !top_k_index || !top_k_weights || !out || (router && !router->logits))
    return fail(MOE_ERR_NULL, "hidden_states / router_logits / top_k_index / top_k_weights / out is NULL");
  if (stat && !opt->act_scales) return fail(MOE_ERR_NULL, "static activation scales requested but act_scales is NULL");
  if (stat && (const void*)out == opt->act_scales) return fail(MOE_ERR_UNSUPPORTED, "out must not alias an input");
  if ((const void*)out == (const void*)hidden_states || (const void*)out == (const void*)top_k_index ||
      (const void*)out == (const void*)top_k_weights)
    return fail(MOE_ERR_UNSUPPORTED, "out must not alias an input");
  if (router) {
    const void* o[] = {top_k_index, top_k_weights, out};
    for (const void* q : o)
      if (q == (const void*)router->logits || q == (const void*)hidden_states)
        return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias inputs");
    if ((const void*)top_k_index == (const void*)top_k_weights || (const void*)top_k_index == (const void*)out ||
        (const void*)top_k_weights == (const void*)out)
      return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias one another");
  }
  const FwdLayout L = fwd_layout(T, k, w->E, w->H, w->I, w->fmt);
  if (!ws || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed", ws ? ws_bytes : (size_t)0, L.total);
  int dev, cus;
  if ((st = check_device(stream, &dev, &cus)) != MOE_OK) return st;
  const moe_debug* dbg = opt ? opt->debug : nullptr;
  if ((st = check_ptrs(dev, {{hidden_states, "hidden_states"},
                             {top_k_index, "top_k_index"},
                             {top_k_weights, "top_k_weights"},
                             {out, "out"},
                             {w->w13, "w13"},
                             {w->w13_scale, "w13_scale"},
                             {w->w2, "w2"},
                             {w->w2_scale, "w2_scale"},
                             {ws_is_scratch ? nullptr : ws, "workspace"},
                             {opt ? opt->invalid_count : nullptr, "invalid_count"},
                             {stat ? opt->act_scales : nullptr, "act_scales"},
                             {dbg ? dbg->sorted_slot : nullptr, "debug.sorted_slot"},
                             {dbg ? dbg->expert_offsets : nullptr, "debug.expert_offsets"},
                             {dbg ? dbg->act_codes : nullptr, "debug.act_codes"},
                             {dbg ? dbg->act_scales : nullptr, "debug.act_scales"},
                             {dbg ? dbg->h_codes : nullptr, "debug.h_codes"},
                             {dbg ? dbg->h_scales : nullptr, "debug.h_scales"}})) != MOE_OK)
    return st;

  const int E = w->E, H = w->H, I = w->I;
  const int32_t S = T * k;
  uint8_t* base = (uint8_t*)ws;
  int32_t* sorted_slot = (int32_t*)(base + L.sorted_slot);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  uint8_t* act_codes = base + L.act_codes;
  void* act_scales = base + L.act_scales;
  uint8_t* h_codes = base + L.h_codes;
  void* h_scales = base + L.h_scales;
  uint16_t* slot_out = (uint16_t*)(base + L.slot_out);
  const int32_t expert_begin = opt ? opt->expert_begin : 0;

  int32_t* sched = (int32_t*)(base + L.sched);
  if (router && (st = check_ptr(router->logits, dev, "router_logits")) != MOE_OK) return st;
  const bool bf = w->fmt == MOE_FMT_BF16;
  hipError_t he;
  if (bf)  // nothing to quantize: the gate_up GEMM gathers bf16 rows of hidden_states
    he = moe::launch_route_sort_zero(router, top_k_index, T, k, E, expert_begin, sorted_slot, offsets, nullptr,
                                     opt ? opt->invalid_count : nullptr, base + L.sort_ws, sched,
                                     2 * MOE_TILE_COUNTERS_BYTES / 4, stream);
  else {
    const moe::StaticScales sts{stat ? opt->act_scales : nullptr, stat ? opt->act_scales_row_stride : 0};
    he = moe::launch_route_sort_and_quant(router, top_k_index, T, k, E, expert_begin, sorted_slot, offsets,
                                          opt ? opt->invalid_count : nullptr, base + L.sort_ws, hidden_states, T, H,
                                          w->fmt, act_codes, act_scales, sched, 2 * MOE_TILE_COUNTERS_BYTES / 4,
                                          stream, L.sorted_scales ? base + L.act_scales_sorted : nullptr,
                                          stat ? &sts : nullptr);
  }
  if (he != hipSuccess) return hip_status(he, "route sort / quant launch");

  moe::GemmParams p1{};
  p1.a_codes = bf ? (const uint8_t*)hidden_states : act_codes;
  p1.a_scales = bf ? nullptr : act_scales;
  p1.a_row_index = sorted_slot;
  p1.a_row_div = k;
  p1.a_rows = T;
  p1.offsets = offsets;
  p1.E = E;
  p1.b_codes = w->w13;
  p1.b_scales = w->w13_scale;
  p1.N = 2 * I;
  p1.K = H;
  p1.max_rows = S;
  p1.h_codes = h_codes;
  p1.sched = sched;
  p1.h_scales = h_scales;
  p1.has_limit = has_limit ? 1 : 0;
  p1.limit = has_limit ? opt->swiglu_limit : 0.0f;
  p1.a_scales_sorted = L.sorted_scales ? base + L.act_scales_sorted : nullptr;
  he = launch_gemm(p1, w->fmt, moe::kEpiSwiGLUQuant, true, cus, stream);
  if (he != hipSuccess) return hip_status(he, "gate_up gemm launch");

  moe::GemmParams p2{};
  p2.a_codes = h_codes;
  p2.a_scales = h_scales;
  p2.a_row_index = nullptr;
  p2.a_row_div = 1;
  p2.a_rows = S;
  p2.offsets = offsets;
  p2.E = E;
  p2.b_codes = w->w2;
  p2.b_scales = w->w2_scale;
  p2.N = H;
  p2.K = I;
  p2.max_rows = S;
  p2.slot_out = slot_out;
  p2.top_k_weights = top_k_weights;
  p2.slot_of_row = sorted_slot;
  p2.sched = sched + MOE_TILE_COUNTERS_BYTES / 4;
  he = launch_gemm(p2, w->fmt, moe::kEpiWeightedScatter, false, cus, stream);
  if (he != hipSuccess) return hip_status(he, "down gemm launch");

  he = moe::launch_combine(slot_out, top_k_index, T, k, H, E, expert_begin, out, stream);
  if (he != hipSuccess) return hip_status(he, "combine launch");

  if (opt && opt->debug) {
    const moe_debug* d = opt->debug;
    const bool mx = w->fmt == MOE_FMT_MXFP8A_MXFP4W;
    const size_t sc_bytes = mx ? (size_t)T * (H / 32) : 4 * (size_t)T * (H / 128);  // same in either layout
    if ((d->sorted_slot &&
         (he = hipMemcpyAsync(d->sorted_slot, sorted_slot, 4 * (size_t)S, hipMemcpyDeviceToDevice, stream)) !=
             hipSuccess) ||
        (d->expert_offsets &&
         (he = hipMemcpyAsync(d->expert_offsets, offsets, 4 * (size_t)(E + 1), hipMemcpyDeviceToDevice, stream)) !=
             hipSuccess) ||
        (d->act_codes && !bf &&
         (he = hipMemcpyAsync(d->act_codes, act_codes, (size_t)T * H, hipMemcpyDeviceToDevice, stream)) !=
             hipSuccess) ||
        (d->act_scales && !bf &&
         (he = hipMemcpyAsync(d->act_scales, act_scales, sc_bytes, hipMemcpyDeviceToDevice, stream)) != hipSuccess) ||
        (d->h_codes && !bf &&
         (he = hipMemcpyAsync(d->h_codes, h_codes, (size_t)S * I, hipMemcpyDeviceToDevice, stream)) != hipSuccess) ||
        (d->h_scales && !bf &&
         (he = hipMemcpyAsync(d->h_scales, h_scales, mx ? (size_t)S * (I / 32) : 4 * (size_t)S * (I / 128),
                              hipMemcpyDeviceToDevice, stream)) != hipSuccess))
      return hip_status(he, "debug copy");
  }
  return ok();
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_ARCH: return "MOE_ERR_ARCH";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_forward_sorts_scales(int32_t T, int32_t k, moe_format fmt) {
  if (T <= 0 || k < 1 || k > kMaxK || (int64_t)T * k >= (int64_t)1 << 31) return 0;
  return fmt != MOE_FMT_BF16 && valid_fmt(fmt) && moe::route_sort_multiblock(T * k) ? 1 : 0;
}

size_t moe_route_sort_workspace(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || k > kMaxK || E < 1 || E > kMaxE || (int64_t)T * k >= (int64_t)1 << 31) return 0;
  return moe::route_sort_ws_bytes(T * k, E);
}

moe_status moe_route_sort(const int32_t* top_k_index, int32_t T, int32_t k, int32_t E, int32_t expert_begin,
                          int32_t* sorted_slot, int32_t* expert_offsets, int32_t* slot_pos, int32_t* invalid_count,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d < 0", T);
  if (k < 1 || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, %d]", k, kMaxK);
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxE);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must stay below 2^31");
  if (expert_begin < 0) return fail(MOE_ERR_SHAPE, "expert_begin=%d < 0", expert_begin);
  if (!expert_offsets) return fail(MOE_ERR_NULL, "expert_offsets is NULL");
  if (T > 0 && (!top_k_index || !sorted_slot)) return fail(MOE_ERR_NULL, "top_k_index / sorted_slot is NULL");
  const size_t ws_need = moe_route_sort_workspace(T, k, E);
  if (ws_need > 0 && (!ws || ws_bytes < ws_need))
    return fail(MOE_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed", ws ? ws_bytes : (size_t)0, ws_need);
  if (T > 0 && ((const void*)top_k_index == (const void*)sorted_slot ||
                (const void*)top_k_index == (const void*)slot_pos))
    return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias top_k_index");
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs(dev, {{top_k_index, "top_k_index"},
                             {sorted_slot, "sorted_slot"},
                             {expert_offsets, "expert_offsets"},
                             {slot_pos, "slot_pos"},
                             {invalid_count, "invalid_count"}})) != MOE_OK)
    return st;
  if (ws_need > 0 && (st = check_ptr(ws, dev, "workspace")) != MOE_OK) return st;
  st = hip_status(moe::launch_route_sort(nullptr, top_k_index, T, k, E, expert_begin, sorted_slot, expert_offsets,
                                         slot_pos, invalid_count, ws, stream),
                  "route sort launch");
  return st == MOE_OK ? ok() : st;
}

size_t moe_route_topk_workspace(int32_t T, int32_t k, int32_t E) { return moe_route_sort_workspace(T, k, E); }

moe_status moe_route_topk(const float* router_logits, int32_t T, int32_t n_experts, int32_t k, int32_t renormalize,
                          int32_t* top_k_index, float* top_k_weights, int32_t E, int32_t expert_begin,
                          int32_t* sorted_slot, int32_t* expert_offsets, int32_t* slot_pos, int32_t* invalid_count,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d < 0", T);
  if (n_experts < 1 || n_experts > kMaxE) return fail(MOE_ERR_SHAPE, "n_experts=%d outside [1, %d]", n_experts, kMaxE);
  if (k < 1 || k > kMaxK || k > n_experts)
    return fail(MOE_ERR_SHAPE, "k=%d outside [1, min(%d, n_experts=%d)]", k, kMaxK, n_experts);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must stay below 2^31");
  const bool sort = expert_offsets != nullptr;
  if (!sort && (sorted_slot || slot_pos))
    return fail(MOE_ERR_NULL, "sorted_slot / slot_pos given without expert_offsets");
  if (sort && T > 0 && !sorted_slot) return fail(MOE_ERR_NULL, "sorted_slot is NULL");
  if (sort && (E < 1 || E > kMaxE)) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxE);
  if (sort && expert_begin < 0) return fail(MOE_ERR_SHAPE, "expert_begin=%d < 0", expert_begin);
  if (T == 0) {
    if (!sort) return ok();
  } else if (!router_logits || !top_k_index || !top_k_weights) {
    return fail(MOE_ERR_NULL, "router_logits / top_k_index / top_k_weights is NULL");
  }
  const size_t ws_need = sort ? moe_route_sort_workspace(T, k, E) : 0;
  if (ws_need > 0 && (!ws || ws_bytes < ws_need))
    return fail(MOE_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed", ws ? ws_bytes : (size_t)0, ws_need);
  const void* outs[] = {top_k_index, top_k_weights, sorted_slot, expert_offsets, slot_pos, invalid_count};
  for (const void* o : outs)
    if (o && T > 0 && o == (const void*)router_logits) return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias router_logits");
  if (T > 0 && ((const void*)top_k_index == (const void*)top_k_weights ||
                (sort && ((const void*)sorted_slot == (const void*)top_k_index ||
                          (const void*)slot_pos == (const void*)top_k_index))))
    return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias one another");
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs(dev, {{router_logits, "router_logits"},
                             {top_k_index, "top_k_index"},
                             {top_k_weights, "top_k_weights"},
                             {sorted_slot, "sorted_slot"},
                             {expert_offsets, "expert_offsets"},
                             {slot_pos, "slot_pos"},
                             {invalid_count, "invalid_count"}})) != MOE_OK)
    return st;
  if (ws_need > 0 && (st = check_ptr(ws, dev, "workspace")) != MOE_OK) return st;
  const moe::RouterArgs r{router_logits, n_experts, renormalize ? 1 : 0, top_k_index, top_k_weights};
  hipError_t he;
  if (sort)
    he = moe::launch_route_sort(T > 0 ? &r : nullptr, top_k_index, T, k, E, expert_begin, sorted_slot, expert_offsets,
                                slot_pos, invalid_count, ws, stream);
  else
    he = moe::launch_router_only(r, T, k, stream);
  st = hip_status(he, "router / route sort launch");
  return st == MOE_OK ? ok() : st;
}

moe_status moe_quant_act(const uint16_t* x, int32_t rows, int32_t H, moe_format fmt, uint8_t* codes, void* scales,
                         hipStream_t stream) {
  if (!valid_fmt(fmt)) return fail(MOE_ERR_UNSUPPORTED, "unknown format %d", (int)fmt);
  if (rows < 0) return fail(MOE_ERR_SHAPE, "rows=%d < 0", rows);
  if (H <= 0 || H % 128) return fail(MOE_ERR_SHAPE, "H=%d must be a positive multiple of 128", H);
  if (rows > 0 && (!x || !codes || !scales)) return fail(MOE_ERR_NULL, "x / codes / scales is NULL");
  if ((const void*)x == (const void*)codes || (const void*)x == scales)
    return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias x");
  if (rows == 0) return ok();
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs(dev, {{x, "x"}, {codes, "codes"}, {scales, "scales"}})) != MOE_OK) return st;
  st = hip_status(moe::launch_quant_act(x, rows, H, (int)fmt, codes, scales, stream), "quant launch");
  return st == MOE_OK ? ok() : st;
}

moe_status moe_quant_act_static(const uint16_t* x, int32_t rows, int32_t H, moe_format fmt, const void* act_scales,
                                int32_t row_stride, uint8_t* codes, void* scales, hipStream_t stream) {
  if (!valid_fmt(fmt)) return fail(MOE_ERR_UNSUPPORTED, "unknown format %d", (int)fmt);
  if (fmt == MOE_FMT_BF16) return fail(MOE_ERR_UNSUPPORTED, "MOE_FMT_BF16 has no activation quantization");
  if (rows < 0) return fail(MOE_ERR_SHAPE, "rows=%d < 0", rows);
  if (H <= 0 || H % 128) return fail(MOE_ERR_SHAPE, "H=%d must be a positive multiple of 128", H);
  const int32_t nb = H / (fmt == MOE_FMT_FP8_B128 ? 128 : 32);
  if (row_stride < 0 || (row_stride > 0 && row_stride < nb))
    return fail(MOE_ERR_SHAPE, "row_stride=%d: 0 or at least one row of %d block scales", row_stride, nb);
  if (rows > 0 && (!x || !codes || !scales || !act_scales)) return fail(MOE_ERR_NULL, "x / act_scales / codes / scales is NULL");
  if ((const void*)x == (const void*)codes || (const void*)x == scales || act_scales == (const void*)codes ||
      act_scales == scales)
    return fail(MOE_ERR_UNSUPPORTED, "outputs must not alias the inputs");
  if (rows == 0) return ok();
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs(dev, {{x, "x"}, {act_scales, "act_scales"}, {codes, "codes"}, {scales, "scales"}})) != MOE_OK)
    return st;
  const moe::StaticScales sts{act_scales, row_stride};
  st = hip_status(moe::launch_quant_act(x, rows, H, (int)fmt, codes, scales, stream, &sts), "quant launch");
  return st == MOE_OK ? ok() : st;
}

size_t moe_prepared_weights_size(moe_format fmt, int32_t E, int32_t H, int32_t I) {
  if (!valid_fmt(fmt) || E < 1 || H <= 0 || I <= 0 || H % 128 || I % 128) return 0;
  const size_t A = 256;
  const size_t e = (size_t)E, h = (size_t)H, i = (size_t)I;
  if (fmt == MOE_FMT_BF16)  // down weight rows padded to whole 256-row tiles
    return align_up(e * 2 * i * h * 2, A) + align_up(e * ((h + 255) / 256 * 256) * i * 2, A);
  if (fmt == MOE_FMT_FP8_B128) {
    const size_t nt2 = (h + 255) / 256;
    return align_up(e * 2 * i * h, A) + align_up(4 * e * (2 * i / 128) * (h / 128), A) +
           align_up(e * nt2 * 256 * i, A) + align_up(4 * e * (h / 128) * (i / 128), A);
  }
  const size_t rows2 = (h + 255) / 256 * 256;  // down weight rows padded to whole tiles
  return align_up(e * 2 * i * h / 2, A) + align_up(e * 2 * i * (h / 32), A) + align_up(e * rows2 * i / 2, A) +
         align_up(e * rows2 * (i / 32), A);
}

moe_status moe_prepare_weights(moe_format fmt, moe_layout layout, int32_t E, int32_t H, int32_t I,
                               const void* gate_up, const void* gate_up_scale, const void* down,
                               const void* down_scale, void* prepared, size_t prepared_bytes, moe_weights* out,
                               hipStream_t stream) {
  if (!out) return fail(MOE_ERR_NULL, "output descriptor is NULL");
  if (!valid_fmt(fmt)) return fail(MOE_ERR_UNSUPPORTED, "unknown format %d", (int)fmt);
  if (layout != MOE_LAYOUT_NT && layout != MOE_LAYOUT_NN) return fail(MOE_ERR_UNSUPPORTED, "unknown layout");
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_SHAPE, "E=%d outside [1, %d]", E, kMaxE);
  if (H <= 0 || I <= 0 || H % 128 || I % 128)
    return fail(MOE_ERR_SHAPE, "H=%d and I=%d must be positive multiples of 128", H, I);
  if ((int64_t)2 * I * H >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "one expert's weight must stay below 2^31");
  const bool bf = fmt == MOE_FMT_BF16;
  if (!gate_up || !down || (!bf && (!gate_up_scale || !down_scale)))
    return fail(MOE_ERR_NULL, "a weight pointer is NULL");
  if (layout == MOE_LAYOUT_NN && fmt == MOE_FMT_MXFP8A_MXFP4W)
    return fail(MOE_ERR_UNSUPPORTED, "the nn layout is accepted for FP8_B128 and BF16 weights only");
  if (!prepared) return fail(MOE_ERR_NULL, "prepared buffer is NULL");
  const size_t need = moe_prepared_weights_size(fmt, E, H, I);
  if (prepared_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "prepared buffer holds %zu bytes, %zu needed", prepared_bytes, need);
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  if ((st = check_ptrs(dev, {{gate_up, "gate_up"},
                             {bf ? nullptr : gate_up_scale, "gate_up_scale"},
                             {down, "down"},
                             {bf ? nullptr : down_scale, "down_scale"},
                             {prepared, "prepared"}})) != MOE_OK)
    return st;
  const size_t A = 256;
  const size_t e = E, h = H, i = I;
  if (bf) {
    // bf16 weights tiled like the FP8 codes, two bytes per element
    uint8_t* q13 = (uint8_t*)prepared;
    uint8_t* q2 = q13 + align_up(e * 2 * i * h * 2, A);
    hipError_t he;
    const bool nn = layout == MOE_LAYOUT_NN;
    if ((he = moe::launch_tile_weight_bf16((const uint16_t*)gate_up, nn, true, E, 2 * I, H, (uint16_t*)q13,
                                           stream)) != hipSuccess ||
        (he = moe::launch_tile_weight_bf16((const uint16_t*)down, nn, false, E, H, I, (uint16_t*)q2, stream)) !=
            hipSuccess)
      return hip_status(he, "weight tiling");
    moe_weights w{};
    w.fmt = fmt;
    w.E = E;
    w.H = H;
    w.I = I;
    w.w13 = q13;
    w.w13_scale = nullptr;
    w.w2 = q2;
    w.w2_scale = nullptr;
    *out = w;
    return ok();
  }
  const bool mx = fmt == MOE_FMT_MXFP8A_MXFP4W;
  const size_t b13 = mx ? e * 2 * i * h / 2 : e * 2 * i * h;
  const size_t b13s = mx ? e * 2 * i * (h / 32) : 4 * e * (2 * i / 128) * (h / 128);
  const size_t rows2 = (h + 255) / 256 * 256;
  const size_t b2 = mx ? e * rows2 * i / 2 : e * rows2 * i;
  const size_t b2s = mx ? e * rows2 * (i / 32) : 4 * e * (h / 128) * (i / 128);
  uint8_t* p13 = (uint8_t*)prepared;
  uint8_t* p13s = p13 + align_up(b13, A);
  uint8_t* p2 = p13s + align_up(b13s, A);
  uint8_t* p2s = p2 + align_up(b2, A);
  hipError_t he = hipSuccess;
  if (mx) {
    if ((he = moe::launch_tile_weight_mx((const uint8_t*)gate_up, (const uint8_t*)gate_up_scale, true, E, 2 * I, H,
                                         p13, p13s, stream)) != hipSuccess ||
        (he = moe::launch_tile_weight_mx((const uint8_t*)down, (const uint8_t*)down_scale, false, E, H, I, p2, p2s,
                                         stream)) != hipSuccess)
      return hip_status(he, "weight tiling");
  } else {
    const bool nn = layout == MOE_LAYOUT_NN;
    if ((he = moe::launch_tile_weight_fp8((const uint8_t*)gate_up, nn, true, E, 2 * I, H, p13, stream)) != hipSuccess ||
        (he = moe::launch_tile_weight_fp8((const uint8_t*)down, nn, false, E, H, I, p2, stream)) != hipSuccess)
      return hip_status(he, "weight tiling");
    if (!nn) {
      if ((he = hipMemcpyAsync(p13s, gate_up_scale, b13s, hipMemcpyDeviceToDevice, stream)) != hipSuccess ||
          (he = hipMemcpyAsync(p2s, down_scale, b2s, hipMemcpyDeviceToDevice, stream)) != hipSuccess)
        return hip_status(he, "scale copy");
    } else {
      // scales [E, H/128, 2I/128] -> [E, 2I/128, H/128] and [E, I/128, H/128] -> [E, H/128, I/128]
      if ((he = moe::launch_transpose_f32((const float*)gate_up_scale, (float*)p13s, E, H / 128, 2 * I / 128,
                                          stream)) != hipSuccess ||
          (he = moe::launch_transpose_f32((const float*)down_scale, (float*)p2s, E, I / 128, H / 128, stream)) !=
              hipSuccess)
        return hip_status(he, "scale transpose");
    }
  }
  moe_weights w;
  w.fmt = fmt;
  w.E = E;
  w.H = H;
  w.I = I;
  w.w13 = p13;
  w.w13_scale = p13s;
  w.w2 = p2;
  w.w2_scale = p2s;
  *out = w;
  return ok();
}

moe_status moe_grouped_gemm(const moe_gemm_args* args, hipStream_t stream) {
  moe_status st = validate_gemm(args);
  if (st != MOE_OK) return st;
  if (args->max_rows == 0) return ok();
  int dev, cus;
  if ((st = check_device(stream, &dev, &cus)) != MOE_OK) return st;
  // every pointer this launch dereferences: the weight it multiplies by, the
  // operand and the outputs and inputs of its epilogue
  const moe_weights* wt = args->weights;
  const bool bf = wt->fmt == MOE_FMT_BF16;
  const moe_epilogue epi = args->epilogue;
  if ((st = check_ptrs(dev, {{args->which == 0 ? wt->w13 : wt->w2, args->which == 0 ? "weights.w13" : "weights.w2"},
                             {bf ? nullptr : (args->which == 0 ? wt->w13_scale : wt->w2_scale),
                              args->which == 0 ? "weights.w13_scale" : "weights.w2_scale"},
                             {args->a_codes, "a_codes"},
                             {bf ? nullptr : args->a_scales, "a_scales"},
                             {args->a_row_index, "a_row_index"},
                             {args->expert_offsets, "expert_offsets"},
                             {epi == MOE_EPI_STORE_F32 ? args->c_f32 : nullptr, "c_f32"},
                             {epi == MOE_EPI_SWIGLU_QUANT ? args->h_codes : nullptr, "h_codes"},
                             {epi == MOE_EPI_SWIGLU_QUANT && !bf ? args->h_scales : nullptr, "h_scales"},
                             {epi == MOE_EPI_WEIGHTED_SCATTER ? args->slot_out : nullptr, "slot_out"},
                             {epi == MOE_EPI_WEIGHTED_SCATTER ? args->top_k_weights : nullptr, "top_k_weights"},
                             {epi == MOE_EPI_WEIGHTED_SCATTER ? args->slot_of_row : nullptr, "slot_of_row"},
                             {args->tile_counters, "tile_counters"},
                             {bf ? nullptr : args->a_scales_sorted, "a_scales_sorted"}})) != MOE_OK)
    return st;
  const moe::GemmParams p = to_params(args);
  const bool paired = args->which == 0;
  st = hip_status(launch_gemm(p, args->weights->fmt, (int)args->epilogue, paired, cus, stream),
                  "grouped gemm launch");
  return st == MOE_OK ? ok() : st;
}

size_t moe_experts_forward_workspace(int32_t T, int32_t k, const moe_weights* w) {
  if (!w || T < 0 || k < 1 || !valid_fmt(w->fmt) || w->E < 1 || w->H <= 0 || w->I <= 0) return 0;
  return fwd_layout(T, k, w->E, w->H, w->I, w->fmt).total;
}

moe_status moe_experts_forward(const moe_weights* w, const uint16_t* hidden_states, const int32_t* top_k_index,
                               const float* top_k_weights, int32_t T, int32_t k, const moe_options* opt,
                               uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return forward_impl(w, hidden_states, nullptr, top_k_index, top_k_weights, T, k, opt, out, ws, ws_bytes, stream);
}

moe_status moe_experts_forward_noalloc(const moe_weights* w, const uint16_t* hidden_states,
                                       const int32_t* top_k_index, const float* top_k_weights, int32_t T, int32_t k,
                                       const moe_options* opt, uint16_t* out, hipStream_t stream) {
  // host-only checks first, so a refused call touches no device state
  moe_status st = validate_weights(w);
  if (st != MOE_OK) return st;
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d < 0", T);
  if (k < 1 || k > kMaxK) return fail(MOE_ERR_SHAPE, "k=%d outside [1, %d]", k, kMaxK);
  if ((int64_t)T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must stay below 2^31");
  if (T == 0) return forward_impl(w, hidden_states, nullptr, top_k_index, top_k_weights, T, k, opt, out, nullptr, 0,
                                  stream);
  const size_t need = fwd_layout(T, k, w->E, w->H, w->I, w->fmt).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this forward needs %zu bytes of workspace; the no-allocation entry point holds %zu per GPU (use "
                "moe_experts_forward with a caller workspace)",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  int dev, cus;
  if ((st = check_device(stream, &dev, &cus)) != MOE_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(dev, &ws)) != MOE_OK) return st;
  return forward_impl(w, hidden_states, nullptr, top_k_index, top_k_weights, T, k, opt, out, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, stream, true);
}

moe_status moe_probe_mfma_rate(int32_t kind, int32_t iters, double* tflops, double* sclk_ghz, hipStream_t stream) {
  if (!tflops || !sclk_ghz) return fail(MOE_ERR_NULL, "tflops / sclk_ghz are NULL");
  if (kind < 0 || kind > 4) return fail(MOE_ERR_UNSUPPORTED, "probe kind %d outside [0, 4]", (int)kind);
  if (iters < 1 || iters > (1 << 24)) return fail(MOE_ERR_SHAPE, "iters=%d outside [1, 2^24]", (int)iters);
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  const int grid = cus, threads = moe::probe_threads();
  iters = (iters + 1) & ~1;  // the probe runs its rounds in pairs
  float* sink = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  std::vector<unsigned long long> h_clk(2 * (size_t)grid);
  float ms = 0.0f;
  hipError_t he = hipMalloc(&sink, sizeof(float) * (size_t)grid * threads);
  if (he == hipSuccess) he = hipMalloc(&clk, sizeof(unsigned long long) * 2 * (size_t)grid);
  if (he == hipSuccess) he = hipEventCreate(&e0);
  if (he == hipSuccess) he = hipEventCreate(&e1);
  // a short warm-up launch, then the timed one
  if (he == hipSuccess) he = moe::launch_mfma_probe(kind, iters / 8 + 1, grid, sink, clk, stream);
  if (he == hipSuccess) he = hipEventRecord(e0, stream);
  if (he == hipSuccess) he = moe::launch_mfma_probe(kind, iters, grid, sink, clk, stream);
  if (he == hipSuccess) he = hipEventRecord(e1, stream);
  if (he == hipSuccess) he = hipEventSynchronize(e1);
  if (he == hipSuccess) he = hipEventElapsedTime(&ms, e0, e1);
  if (he == hipSuccess)
    he = hipMemcpy(h_clk.data(), clk, sizeof(unsigned long long) * h_clk.size(), hipMemcpyDeviceToHost);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (sink) (void)hipFree(sink);
  if (clk) (void)hipFree(clk);
  if (he != hipSuccess) return hip_status(he, "mfma probe");
  if (!(ms > 0.0f)) return fail(MOE_ERR_HIP, "mfma probe: no elapsed time");
  double shader = 0.0, real = 0.0;
  for (int b = 0; b < grid; ++b) {
    shader += (double)h_clk[2 * b];
    real += (double)h_clk[2 * b + 1];
  }
  const double flops = (double)grid * (threads / 64) * (double)iters * (double)moe::probe_mfmas_per_round(kind) *
                       (double)moe::probe_flops_per_mfma(kind);
  *tflops = flops / ((double)ms * 1e-3) / 1e12;
  *sclk_ghz = real > 0.0 ? shader / real * 0.1 : 0.0;  // the real-time counter ticks at 100 MHz
  return ok();
}

moe_status moe_clock_stamp(uint64_t* stamps, int32_t n, hipStream_t stream) {
  if (!stamps) return fail(MOE_ERR_NULL, "stamps is NULL");
  if (n < 1 || n > kMaxClockStamps) return fail(MOE_ERR_SHAPE, "n=%d outside [1, %d]", (int)n, kMaxClockStamps);
  int dev, cus;
  moe_status st = check_device(stream, &dev, &cus);
  if (st != MOE_OK) return st;
  if ((st = check_ptr(stamps, dev, "stamps")) != MOE_OK) return st;
  const hipError_t he = moe::launch_clock_stamp(reinterpret_cast<unsigned long long*>(stamps), n, stream);
  if (he != hipSuccess) return hip_status(he, "clock stamp");
  return ok();
}

moe_status moe_experts_forward_from_logits(const moe_weights* w, const uint16_t* hidden_states,
                                           const float* router_logits, int32_t T, int32_t n_experts, int32_t k,
                                           int32_t renormalize, const moe_options* opt, int32_t* top_k_index,
                                           float* top_k_weights, uint16_t* out, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  const moe::RouterArgs r{router_logits, n_experts, renormalize ? 1 : 0, top_k_index, top_k_weights};
  return forward_impl(w, hidden_states, &r, top_k_index, top_k_weights, T, k, opt, out, ws, ws_bytes, stream);
}

}  // extern "C"
