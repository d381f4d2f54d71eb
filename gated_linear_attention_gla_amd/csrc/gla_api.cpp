// gla_api.cpp -- C ABI of libgla.so: argument validation and pass dispatch.
//
// Everything here runs on the host.  Each entry point checks all of its
// arguments before touching the HIP runtime, so a rejected call enqueues
// nothing (and can be exercised on a machine without a GPU).
//
// Backward passes.  For L = sum_t <dO_t, o_t> + <dS_T, S_T> (page "Beyond
// the KV cache ...", section "Challenge 3": the backward runs through the
// sequential state updates), with G_t = dL/dS_t:
//   dq_t = S_t dO_t                       -- forward-time recurrence on S^T
//   G_t  = lam G_{t+1} + q_t dO_t^T,  G_T = dS_T + q_T dO_T^T
//   dv_t = G_t^T k_t,  dk_t = G_t v_t,  dS_0 = lam G_1
// Each of dq, dv, dk is one chunked recurrence of the same form as the
// forward with the roles of (q, k, v) permuted:
//   dq: query dO, key v,  value k,  state S^T (starts at S0^T), forward time
//   dv: query k,  key q,  value dO, state G   (starts at dS_T), reverse time
//   dk: query v,  key dO, value q,  state G^T (starts at dS_T^T), reverse time
// and the final state of the dv pass is dS0.
//
// Segment split (page section "Challenge 1": the chunks are independent, only
// the state chain is serial).  When too few (b, h) units exist to fill the
// GPU, a pass splits the tokens into segments: a state pass computes every
// segment's end state from a zero start into the workspace, then each
// segment's full pass starts from lam^len-weighted sums of the earlier ones.
#include "../../include/gla.h"
#include "gla_internal.h"

#include <stdint.h>

#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

// Device scratch of gla_chunk_fwd_noalloc: the segment end states of its
// segment split (the same use as gla_chunk_fwd's workspace).  Every GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress (noalloc_scratch below) and only
// that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[GLA_NOALLOC_SCRATCH_BYTES];

using gla::ChunkArgs;
using gla::DecodeArgs;

namespace {

int esize(int32_t dt) { return dt == GLA_F32 ? 4 : 2; }
bool dtype_ok(int32_t dt) { return dt == GLA_F32 || dt == GLA_BF16; }

// Row starts of a (b, h, t) view must be 16-byte aligned; strides that are
// never stepped (size-1 dims) are not constrained.  Along t, rows of d
// elements must not overlap (stride_t >= d) and one chunk of rows must span
// less than 2 GiB (the kernels address a chunk tile with 32-bit offsets).
gla_status check_view(const gla_tensor* x, int64_t nb, int64_t nh, int64_t nt, int64_t d,
                      int64_t chunk, bool need_data) {
  if (need_data && x->data == nullptr) return GLA_ERR_NULL;
  if (x->stride_b < 0 || x->stride_h < 0 || x->stride_t < 0) return GLA_ERR_STRIDE;
  const int64_t es = esize(x->dtype);
  if ((reinterpret_cast<uintptr_t>(x->data) & 15u) != 0) return GLA_ERR_STRIDE;
  if (nb > 1 && (x->stride_b * es) % 16 != 0) return GLA_ERR_STRIDE;
  if (nh > 1 && (x->stride_h * es) % 16 != 0) return GLA_ERR_STRIDE;
  if (nt > 1) {
    if ((x->stride_t * es) % 16 != 0 || x->stride_t < d) return GLA_ERR_STRIDE;
    if (x->stride_t > ((int64_t)1 << 31) / (es * chunk)) return GLA_ERR_STRIDE;
  }
  return GLA_OK;
}

bool same(const void* a, const void* b) { return a != nullptr && a == b; }

// A launch covers at most 2^32 - 1 work-items (the dispatch packet's grid
// size is 32 bits): with up to 768 threads per workgroup and two column blocks
// (four workgroups per (b, h) in the backward's paired launch), B * H <= 2^21
// keeps every chunked launch below it.
constexpr int64_t kMaxUnits = (int64_t)1 << 21;

gla_status check_dims(const gla_dims* d) {
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->dk < 1 || d->dv < 1 || d->chunk < 1) return GLA_ERR_SHAPE;
  if (d->B > (int64_t)1 << 24 || d->H > (int64_t)1 << 16 || d->T > (int64_t)1 << 40) return GLA_ERR_SHAPE;
  if (d->B * d->H > kMaxUnits) return GLA_ERR_SHAPE;
  return GLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tokens per segment when a pass is split into nseg segments of whole chunks.
int64_t seg_len_for(int64_t T, int64_t chunk, int nseg) {
  const int64_t nchunks = (T + chunk - 1) / chunk;
  return ((nchunks + nseg - 1) / nseg) * chunk;
}

// Segments of a pass of this shape; the workspace queries take no dtype, so
// they size for the larger count of the two input dtypes (the tiling, and
// with it the count, can differ between them).
int max_segments(const gla_dims* d, int dk, int dv) {
  const int a = gla::chunk_segments(d->B, d->H, d->T, dk, dv, (int)d->chunk, 0);
  const int b = gla::chunk_segments(d->B, d->H, d->T, dk, dv, (int)d->chunk, 1);
  return a > b ? a : b;
}

// Workspace of one segment-split pass: the end state of every (b, h, segment).
size_t pass_workspace(const gla_dims* d, int dk, int dv) {
  const int nseg = max_segments(d, dk, dv);
  if (nseg <= 1) return 0;
  return (size_t)d->B * d->H * nseg * d->dk * d->dv * sizeof(float);
}

// Flags of a one-launch segment split: one 8-byte word per (b, h, column
// block, segment), with at most dv / 16 column blocks.
size_t seg_flag_bytes(const gla_dims* d, int dk, int dv) {
  const int nseg = max_segments(d, dk, dv);
  if (nseg <= 1) return 0;
  return (size_t)d->B * d->H * nseg * ((dv + 15) / 16) * sizeof(unsigned long long);
}

// End states and flags of one pass, rounded to 16 bytes (a second pass's
// region may follow).
size_t pass_bytes(const gla_dims* d, int dk, int dv) {
  return (pass_workspace(d, dk, dv) + seg_flag_bytes(d, dk, dv) + 15) / 16 * 16;
}

// Tag of one call's segment flags: a nonzero 56-bit epoch, distinct per call
// in this process and seeded per process, above the 8 bits that carry the
// XCD id.  Flags left by other calls, processes or earlier users of the
// memory never carry it.
std::atomic<uint64_t> g_seg_epoch{0};
uint64_t next_seg_tag() {
  static const uint64_t seed = [] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return (((uint64_t)rd() << 32) ^ rd() ^ (t * 0x9E3779B97F4A7C15ull));
  }();
  uint64_t e = (seed + g_seg_epoch.fetch_add(1, std::memory_order_relaxed)) & ((1ull << 56) - 1);
  if (e == 0) e = 1;
  return e << 8;
}

// Bound on a workgroup's wait for the earlier segments' states, in ticks of
// the 100 MHz clock: by default 20 us plus 4 us per chunk of a segment (about
// four times a state pass), or the fixed bound set by gla_set_segment_wait.
std::atomic<int32_t> g_seg_wait_us{-1};
uint32_t seg_wait_ticks(int64_t seg_chunks) {
  const int32_t us = g_seg_wait_us.load(std::memory_order_relaxed);
  const int64_t t = us >= 0 ? (int64_t)us * 100 : 2000 + 400 * seg_chunks;
  return (uint32_t)(t > 0xffffffffll ? 0xffffffffll : t);
}

void set_segments(ChunkArgs& a, const gla_dims* d, int dk, int dv, void* ws);

// Segments, end states and flags of a pass whose region starts at ws: the
// one-launch form where the launch allows it.
void set_segments_flags(ChunkArgs& a, const gla_dims* d, int dk, int dv, void* ws) {
  set_segments(a, d, dk, dv, ws);
  if (a.nseg > 1) {
    a.seg_flag = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + pass_workspace(d, dk, dv));
    a.seg_tag = next_seg_tag();
    a.seg_wait = seg_wait_ticks(a.seg_len / d->chunk);
  }
}

void set_segments(ChunkArgs& a, const gla_dims* d, int dk, int dv, void* ws) {
  a.nseg = gla::chunk_segments(d->B, d->H, d->T, dk, dv, (int)d->chunk, a.in_f32);
  a.seg_len = a.nseg > 1 ? seg_len_for(d->T, d->chunk, a.nseg) : (d->T > 0 ? d->T : 1);
  a.seg_state = a.nseg > 1 ? static_cast<float*>(ws) : nullptr;
}

ChunkArgs make_pass(const gla_dims* d, const gla_tensor* qr, const gla_tensor* kr, const gla_tensor* vr,
                    const float* lambda, const float* s_init, int s_init_trans, float* s_final,
                    gla_tensor* out, int reverse) {
  ChunkArgs a{};
  a.q = qr->data;
  a.k = kr->data;
  a.v = vr->data;
  a.sq_b = qr->stride_b; a.sq_h = qr->stride_h; a.sq_t = qr->stride_t;
  a.sk_b = kr->stride_b; a.sk_h = kr->stride_h; a.sk_t = kr->stride_t;
  a.sv_b = vr->stride_b; a.sv_h = vr->stride_h; a.sv_t = vr->stride_t;
  a.o = out->data;
  a.so_b = out->stride_b; a.so_h = out->stride_h; a.so_t = out->stride_t;
  a.lam = lambda;
  a.s_init = s_init;
  a.s_init_trans = s_init_trans;
  a.s_final = s_final;
  a.B = d->B; a.H = d->H; a.T = d->T;
  a.reverse = reverse;
  a.o_f32 = out->dtype == GLA_F32;
  a.in_f32 = qr->dtype == GLA_F32;
  return a;
}

// Device address of `scratch` on the device that runs `stream`, looked up
// once per device with that device current and kept for later calls.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

gla_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return GLA_ERR_HIP;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return GLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return GLA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return GLA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return GLA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GLA_OK;
}

// Validation and launch of the chunked forward.  The segment states live in
// the caller's workspace (ws, ws_bytes), or, with noalloc, in the device's
// static scratch.
gla_status chunk_fwd_impl(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                          const gla_tensor* v, const float* lambda, const float* S0, gla_tensor* o,
                          float* S_T, void* ws, size_t ws_bytes, bool noalloc, void* stream);

}  // namespace

extern "C" {

int gla_abi_version(void) { return GLA_ABI_VERSION; }

const char* gla_status_string(gla_status s) {
  switch (s) {
    case GLA_OK: return "ok";
    case GLA_ERR_NULL: return "a required pointer is NULL";
    case GLA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case GLA_ERR_STRIDE: return "negative stride or misaligned row start (16 bytes required)";
    case GLA_ERR_DTYPE: return "unknown dtype, or q/k/v/dO dtypes differ";
    case GLA_ERR_UNSUPPORTED: return "no compiled kernel for this (dk, dv, chunk, dtype)";
    case GLA_ERR_ALIAS: return "an output aliases an input or another output";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GLA_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

size_t gla_chunk_fwd_workspace(const gla_dims* dims) {
  if (!dims || check_dims(dims) != GLA_OK) return 0;
  return pass_bytes(dims, (int)dims->dk, (int)dims->dv);
}

void gla_set_segment_wait(int32_t microseconds) {
  g_seg_wait_us.store(microseconds < 0 ? -1 : microseconds, std::memory_order_relaxed);
}

size_t gla_chunk_bwd_workspace(const gla_dims* dims) {
  if (!dims || check_dims(dims) != GLA_OK) return 0;
  // the dq and dk passes run together (one region each), then the dv pass
  // reuses the space
  const size_t a = pass_bytes(dims, (int)dims->dk, (int)dims->dv);
  // (the transposed passes may tile shorter than the chunk; sized for both
  // input dtypes, as the query takes none)
  gla_dims dt = *dims;
  size_t b = 0;
  for (int in_f32 = 0; in_f32 < 2; ++in_f32) {
    dt.chunk = gla::bwd_transposed_tile((int)dims->chunk, in_f32);
    const size_t bt = 2 * pass_bytes(&dt, (int)dims->dv, (int)dims->dk);
    b = bt > b ? bt : b;
  }
  return a > b ? a : b;
}

gla_status gla_chunk_fwd(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                         const gla_tensor* v, const float* lambda, const float* S0,
                         gla_tensor* o, float* S_T, void* ws, size_t ws_bytes, void* stream) {
  return chunk_fwd_impl(dims, q, k, v, lambda, S0, o, S_T, ws, ws_bytes, false, stream);
}

gla_status gla_chunk_fwd_noalloc(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                                 const gla_tensor* v, const float* lambda, const float* S0,
                                 gla_tensor* o, float* S_T, void* stream) {
  return chunk_fwd_impl(dims, q, k, v, lambda, S0, o, S_T, nullptr, 0, true, stream);
}

gla_status gla_chunk_bwd(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                         const gla_tensor* v, const float* lambda, const float* S0,
                         const gla_tensor* dO, const float* dS_T, gla_tensor* dq,
                         gla_tensor* dk, gla_tensor* dv, float* dS0, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!dims || !q || !k || !v || !lambda || !dO || !dq || !dk || !dv) return GLA_ERR_NULL;
  gla_status st = check_dims(dims);
  if (st != GLA_OK) return st;
  const int64_t B = dims->B, H = dims->H, T = dims->T;
  if (!dtype_ok(q->dtype) || k->dtype != q->dtype || v->dtype != q->dtype || dO->dtype != q->dtype ||
      !dtype_ok(dq->dtype) || !dtype_ok(dk->dtype) || !dtype_ok(dv->dtype))
    return GLA_ERR_DTYPE;
  const int in_f32 = q->dtype == GLA_F32;
  const int DK = (int)dims->dk, DV = (int)dims->dv, C = (int)dims->chunk;
  if (!gla::chunk_pass_supported(DK, DV, C, in_f32) || !gla::chunk_pass_supported(DV, DK, C, in_f32))
    return GLA_ERR_UNSUPPORTED;
  const bool need = T > 0;
  const gla_tensor* views[] = {q, k, v, dO, dq, dk, dv};
  const int64_t widths[] = {DK, DK, DV, DV, DK, DK, DV};
  for (int i = 0; i < 7; ++i)
    if ((st = check_view(views[i], B, H, T, widths[i], C, need)) != GLA_OK) return st;
  if (!aligned16(S0) || !aligned16(dS_T) || !aligned16(dS0) || !aligned16(lambda)) return GLA_ERR_STRIDE;
  const void* ins[] = {q->data, k->data, v->data, dO->data, lambda, S0, dS_T};
  const void* outs[] = {dq->data, dk->data, dv->data, dS0};
  for (int i = 0; i < 4; ++i) {
    for (const void* p : ins)
      if (same(outs[i], p)) return GLA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (same(outs[i], outs[j])) return GLA_ERR_ALIAS;
  }
  const size_t need_ws = gla_chunk_bwd_workspace(dims);
  if (ws_bytes < need_ws || (need_ws > 0 && (ws == nullptr || !aligned16(ws)))) return GLA_ERR_WORKSPACE;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the transposed passes' tile length (gla::bwd_transposed_tile)
  gla_dims dt = *dims;
  if (DV == 192 && DK == 96) dt.chunk = gla::bwd_transposed_tile(C, in_f32);
  // dq: query dO, key v, value k; state S^T from S0^T; forward time
  ChunkArgs a1 = make_pass(&dt, dO, v, k, lambda, S0, 1, nullptr, dq, 0);
  set_segments_flags(a1, &dt, DV, DK, ws);
  // dk: query v, key dO, value q; state G^T from dS_T^T; reverse time
  ChunkArgs a3 = make_pass(&dt, v, dO, q, lambda, dS_T, 1, nullptr, dk, 1);
  set_segments_flags(a3, &dt, DV, DK, a1.nseg > 1 ? static_cast<char*>(ws) + pass_bytes(&dt, DV, DK) : ws);
  // the two share the transposed shape and run in one launch
  if (gla::launch_chunk_pair(DV, DK, (int)dt.chunk, a1, a3, s) != hipSuccess) return GLA_ERR_HIP;
  // dv (and dS0): query k, key q, value dO; state G from dS_T; reverse time
  ChunkArgs a2 = make_pass(dims, k, q, dO, lambda, dS_T, 0, dS0, dv, 1);
  set_segments_flags(a2, dims, DK, DV, ws);
  if (gla::launch_chunk_pass(DK, DV, C, a2, s) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

// Workspace of the fused decode step: o' (fp32, N*H*dv) and the column
// slices' sums of squares (4 floats per state), when the step runs as column
// slices plus a normalisation kernel; 0 when it runs one workgroup per state.
static size_t decode_fused_ws(int64_t N, int64_t H, int64_t dk, int64_t dv) {
  if (gla::decode_slices(N * H, (int)dk, (int)dv, true, true) <= 1) return 0;
  return (size_t)(N * H) * (size_t)(dv + 4) * sizeof(float);
}

static gla_status decode_impl(int64_t N, int64_t H, int64_t dk, int64_t dv, const gla_tensor* q,
                              const gla_tensor* k, const gla_tensor* v, const float* lambda, float* S,
                              int64_t S_stride_n, const gla_tensor* g, const float* aug, const float* gamma,
                              float eps, gla_tensor* o, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !lambda || !S || !o) return GLA_ERR_NULL;
  // N * H <= 2^24 states: the launch (gla::decode_slices picks three column
  // slices per state while they fit, else one 192-thread workgroup per
  // state) then stays below 2^32 work-items
  if (N < 1 || H < 1 || dk < 1 || dv < 1 || N > (int64_t)1 << 30 || H > (int64_t)1 << 16 ||
      N * H > (int64_t)1 << 24)
    return GLA_ERR_SHAPE;
  if (!dtype_ok(q->dtype) || k->dtype != q->dtype || v->dtype != q->dtype || !dtype_ok(o->dtype))
    return GLA_ERR_DTYPE;
  if (!gla::decode_supported((int)dk, (int)dv)) return GLA_ERR_UNSUPPORTED;
  if (S_stride_n < H * dk * dv) return GLA_ERR_SHAPE;
  gla_status st;
  // decode views are [N, H, d]: stride_b steps n, stride_h steps h
  if ((st = check_view(q, N, H, 1, dk, 1, true)) != GLA_OK) return st;
  if ((st = check_view(k, N, H, 1, dk, 1, true)) != GLA_OK) return st;
  if ((st = check_view(v, N, H, 1, dv, 1, true)) != GLA_OK) return st;
  if ((st = check_view(o, N, H, 1, dv, 1, true)) != GLA_OK) return st;
  if (g) {
    if (!aug || !gamma) return GLA_ERR_NULL;
    if (g->dtype != q->dtype) return GLA_ERR_DTYPE;
    if (!(eps >= 0.0f) || eps > 1e30f) return GLA_ERR_SHAPE;
    if ((st = check_view(g, N, H, 1, dv, 1, true)) != GLA_OK) return st;
    if (!aligned16(aug) || !aligned16(gamma)) return GLA_ERR_STRIDE;
    if (same(o->data, g->data) || same(o->data, aug) || same(o->data, gamma) || same(S, g->data) ||
        same(S, aug) || same(S, gamma))
      return GLA_ERR_ALIAS;
    if (ws != nullptr) {
      const size_t need = decode_fused_ws(N, H, dk, dv);
      if (ws_bytes < need || !aligned16(ws)) return GLA_ERR_WORKSPACE;
      const void* other[] = {q->data, k->data, v->data, g->data, lambda, aug, gamma, S, o->data};
      for (const void* p : other)
        if (same(ws, p)) return GLA_ERR_ALIAS;
      if (need == 0) ws = nullptr;  // this shape runs one workgroup per state
    }
  }
  if (!aligned16(S) || !aligned16(lambda) || (N > 1 && (S_stride_n * 4) % 16 != 0)) return GLA_ERR_STRIDE;
  const void* ins[] = {q->data, k->data, v->data, lambda};
  for (const void* p : ins)
    if (same(o->data, p) || same(S, p)) return GLA_ERR_ALIAS;
  if (same(o->data, S)) return GLA_ERR_ALIAS;

  DecodeArgs a{};
  a.q = q->data; a.k = k->data; a.v = v->data;
  a.sq_n = q->stride_b; a.sq_h = q->stride_h;
  a.sk_n = k->stride_b; a.sk_h = k->stride_h;
  a.sv_n = v->stride_b; a.sv_h = v->stride_h;
  a.lam = lambda;
  a.S = S;
  a.S_stride_n = S_stride_n;
  a.o = o->data;
  a.so_n = o->stride_b; a.so_h = o->stride_h;
  a.N = N; a.H = H;
  a.o_f32 = o->dtype == GLA_F32;
  a.in_f32 = q->dtype == GLA_F32;
  if (g) {
    a.gz = g->data;
    a.sg_n = g->stride_b;
    a.sg_h = g->stride_h;
    a.aug = aug;
    a.gamma = gamma;
    a.eps = eps;
    a.ws = static_cast<float*>(ws);
  }
  if (gla::launch_decode((int)dk, (int)dv, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, const gla_tensor* q,
                           const gla_tensor* k, const gla_tensor* v, const float* lambda,
                           float* S, int64_t S_stride_n, gla_tensor* o, void* stream) {
  return decode_impl(N, H, dk, dv, q, k, v, lambda, S, S_stride_n, nullptr, nullptr, nullptr, 0.0f, o, nullptr, 0,
                     stream);
}

int gla_decode_workgroups_per_state(int64_t N, int64_t H, int64_t dk, int64_t dv, int fused) {
  if (N < 1 || H < 1 || N > (int64_t)1 << 30 || H > (int64_t)1 << 16 || N * H > (int64_t)1 << 24) return 0;
  if (dk < 1 || dv < 1 || dk > 4096 || dv > 4096 || fused < 0 || fused > 2) return 0;
  return gla::decode_slices(N * H, (int)dk, (int)dv, fused != 0, fused == 1);
}

size_t gla_decode_step_fused_workspace(int64_t N, int64_t H, int64_t dk, int64_t dv) {
  if (N < 1 || H < 1 || N > (int64_t)1 << 30 || H > (int64_t)1 << 16 || N * H > (int64_t)1 << 24) return 0;
  if (dk < 1 || dv < 1 || dk > 4096 || dv > 4096) return 0;
  return decode_fused_ws(N, H, dk, dv);
}

gla_status gla_decode_step_fused(int64_t N, int64_t H, int64_t dk, int64_t dv, const gla_tensor* q,
                                 const gla_tensor* k, const gla_tensor* v, const float* lambda, float* S,
                                 int64_t S_stride_n, const gla_tensor* g, const float* aug,
                                 const float* gamma, float eps, gla_tensor* y, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!g) return GLA_ERR_NULL;
  return decode_impl(N, H, dk, dv, q, k, v, lambda, S, S_stride_n, g, aug, gamma, eps, y, ws, ws_bytes, stream);
}

size_t gla_chunk_fwd_fused_workspace(const gla_dims* dims) {
  if (!dims || check_dims(dims) != GLA_OK) return 0;
  // segments of the fused tile (gla::fused_tile), sized for both input dtypes
  int nseg = 1;
  for (int in_f32 = 0; in_f32 < 2; ++in_f32) {
    const int n = gla::chunk_segments_fused(dims->B, dims->H, dims->T, gla::fused_tile((int)dims->chunk, in_f32));
    nseg = n > nseg ? n : nseg;
  }
  if (nseg <= 1) return 0;
  return (size_t)dims->B * dims->H * nseg * dims->dk * dims->dv * sizeof(float);
}

gla_status gla_chunk_fwd_fused(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                               const gla_tensor* v, const float* lambda, const float* S0,
                               const gla_tensor* g, const float* aug, const float* gamma, float eps,
                               gla_tensor* y, float* S_T, void* ws, size_t ws_bytes, void* stream) {
  if (!dims || !q || !k || !v || !g || !y || !lambda || !aug || !gamma) return GLA_ERR_NULL;
  gla_status st = check_dims(dims);
  if (st != GLA_OK) return st;
  if (!(eps >= 0.0f) || eps > 1e30f) return GLA_ERR_SHAPE;
  const int64_t B = dims->B, H = dims->H, T = dims->T;
  if (!dtype_ok(q->dtype) || !dtype_ok(y->dtype) || k->dtype != q->dtype || v->dtype != q->dtype ||
      g->dtype != q->dtype)
    return GLA_ERR_DTYPE;
  const int in_f32 = q->dtype == GLA_F32;
  // the tile length (gla::fused_tile: 128-token chunks tile at 64 tokens)
  const int64_t CT = gla::fused_tile((int)dims->chunk, in_f32);
  if (!gla::chunk_fused_supported((int)dims->dk, (int)dims->dv, (int)CT, in_f32)) return GLA_ERR_UNSUPPORTED;
  const bool need = T > 0;
  const int64_t DK = dims->dk, DV = dims->dv, C = dims->chunk;
  if ((st = check_view(q, B, H, T, DK, C, need)) != GLA_OK) return st;
  if ((st = check_view(k, B, H, T, DK, C, need)) != GLA_OK) return st;
  if ((st = check_view(v, B, H, T, DV, C, need)) != GLA_OK) return st;
  if ((st = check_view(g, B, H, T, DV, C, need)) != GLA_OK) return st;
  if ((st = check_view(y, B, H, T, DV, C, need)) != GLA_OK) return st;
  if (!aligned16(S0) || !aligned16(S_T) || !aligned16(lambda) || !aligned16(aug) || !aligned16(gamma))
    return GLA_ERR_STRIDE;
  const void* ins[] = {q->data, k->data, v->data, g->data, lambda, S0, aug, gamma};
  for (const void* p : ins)
    if (same(y->data, p) || same(S_T, p)) return GLA_ERR_ALIAS;
  if (same(y->data, S_T)) return GLA_ERR_ALIAS;
  const size_t need_ws = gla_chunk_fwd_fused_workspace(dims);
  if (ws_bytes < need_ws || (need_ws > 0 && (ws == nullptr || !aligned16(ws)))) return GLA_ERR_WORKSPACE;

  ChunkArgs a = make_pass(dims, q, k, v, lambda, S0, 0, S_T, y, 0);
  a.nseg = gla::chunk_segments_fused(B, H, T, (int)CT);
  a.seg_len = a.nseg > 1 ? seg_len_for(T, CT, a.nseg) : (T > 0 ? T : 1);
  a.seg_state = a.nseg > 1 ? static_cast<float*>(ws) : nullptr;
  a.gz = g->data;
  a.sg_b = g->stride_b; a.sg_h = g->stride_h; a.sg_t = g->stride_t;
  a.aug = aug;
  a.gamma = gamma;
  a.eps = eps;
  if (gla::launch_chunk_fused((int)DK, (int)DV, (int)CT, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_chunk_fwd_varlen(int64_t N, int64_t H, int64_t total_T, int64_t dk, int64_t dv,
                                int64_t chunk, const gla_tensor* q, const gla_tensor* k,
                                const gla_tensor* v, const int32_t* cu_seqlens, const float* lambda,
                                float* pool, int64_t num_slots, int64_t pool_stride_n,
                                const int32_t* slots, const int32_t* has_state, gla_tensor* o,
                                void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens || !lambda || !pool) return GLA_ERR_NULL;
  if (N < 1 || H < 1 || total_T < 0 || num_slots < 1 || N > ((int64_t)1 << 24) || H > ((int64_t)1 << 16) ||
      N * H > kMaxUnits || total_T > ((int64_t)1 << 31) - 1 || num_slots > ((int64_t)1 << 31))
    return GLA_ERR_SHAPE;
  if (!dtype_ok(q->dtype) || !dtype_ok(o->dtype) || k->dtype != q->dtype || v->dtype != q->dtype)
    return GLA_ERR_DTYPE;
  const int in_f32 = q->dtype == GLA_F32;
  if (!gla::chunk_pass_supported((int)dk, (int)dv, (int)chunk, in_f32)) return GLA_ERR_UNSUPPORTED;
  if (pool_stride_n < H * dk * dv) return GLA_ERR_SHAPE;
  gla_status st;
  // packed [total_T, H, d] views: stride_t steps tokens, stride_h heads
  const bool need = total_T > 0;
  if ((st = check_view(q, 1, H, total_T, dk, chunk, need)) != GLA_OK) return st;
  if ((st = check_view(k, 1, H, total_T, dk, chunk, need)) != GLA_OK) return st;
  if ((st = check_view(v, 1, H, total_T, dv, chunk, need)) != GLA_OK) return st;
  if ((st = check_view(o, 1, H, total_T, dv, chunk, need)) != GLA_OK) return st;
  if (!aligned16(pool) || !aligned16(lambda) || (num_slots > 1 && (pool_stride_n * 4) % 16 != 0))
    return GLA_ERR_STRIDE;
  const void* ins[] = {q->data, k->data, v->data, lambda, cu_seqlens, slots, has_state};
  for (const void* p : ins)
    if (same(o->data, p) || same(pool, p)) return GLA_ERR_ALIAS;
  if (same(o->data, pool)) return GLA_ERR_ALIAS;

  const gla_dims dims{N, H, total_T, dk, dv, chunk};
  ChunkArgs a = make_pass(&dims, q, k, v, lambda, nullptr, 0, nullptr, o, 0);
  a.sq_b = a.sk_b = a.sv_b = a.so_b = 0;
  a.nseg = 1;
  a.seg_len = total_T > 0 ? total_T : 1;
  a.seg_state = nullptr;
  a.cu = cu_seqlens;
  a.pool = pool;
  a.pool_stride_n = pool_stride_n;
  a.num_slots = num_slots;
  a.slots = slots;
  a.has_state = has_state;
  if (gla::launch_chunk_pass((int)dk, (int)dv, (int)chunk, a, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

// ---------------------------------------------------------------- convolution
// [B, T, D] activation views for the convolution: stride_b over sequences,
// stride_t over tokens, channels contiguous; stride_h is not used.
static gla_status check_act(const gla_tensor* x, int64_t nb, int64_t nt, int64_t D) {
  if (x->data == nullptr) return GLA_ERR_NULL;
  if (!dtype_ok(x->dtype)) return GLA_ERR_DTYPE;
  if (x->stride_b < 0 || x->stride_t < 0) return GLA_ERR_STRIDE;
  const int64_t es = esize(x->dtype);
  if (!aligned16(x->data)) return GLA_ERR_STRIDE;
  if (nb > 1 && (x->stride_b * es) % 16 != 0) return GLA_ERR_STRIDE;
  if (nt > 1 && ((x->stride_t * es) % 16 != 0 || x->stride_t < D)) return GLA_ERR_STRIDE;
  return GLA_OK;
}

static bool conv_dims_ok(int64_t D) { return D >= 8 && D % 8 == 0 && D <= ((int64_t)1 << 24); }

gla_status gla_conv1d_fwd(int64_t B, int64_t T, int64_t D, const gla_tensor* x, const float* w,
                          const float* bias, const float* state_in, gla_tensor* y, float* state_out,
                          void* stream) {
  if (!x || !w || !y) return GLA_ERR_NULL;
  if (B < 1 || T < 0 || !conv_dims_ok(D) || B > ((int64_t)1 << 24) || T > ((int64_t)1 << 40))
    return GLA_ERR_SHAPE;
  if (gla::conv_fwd_blocks(B, T, D) > (int64_t)0xFFFFFFFF / gla::conv_fwd_threads()) return GLA_ERR_SHAPE;
  gla_status st;
  if (T > 0) {
    if ((st = check_act(x, B, T, D)) != GLA_OK) return st;
    if ((st = check_act(y, B, T, D)) != GLA_OK) return st;
  } else if (!dtype_ok(x->dtype) || !dtype_ok(y->dtype)) {
    return GLA_ERR_DTYPE;
  }
  if (!aligned16(w) || !aligned16(bias) || !aligned16(state_in) || !aligned16(state_out))
    return GLA_ERR_STRIDE;
  const void* ins[] = {x->data, w, bias, state_in};
  for (const void* p : ins)
    if (same(y->data, p) || same(state_out, p)) return GLA_ERR_ALIAS;
  if (same(y->data, state_out)) return GLA_ERR_ALIAS;

  gla::ConvArgs a{};
  a.x = x->data; a.sx_b = x->stride_b; a.sx_t = x->stride_t;
  a.w = w; a.bias = bias; a.state_in = state_in;
  a.y = y->data; a.sy_b = y->stride_b; a.sy_t = y->stride_t;
  a.state_out = state_out;
  a.B = B; a.T = T; a.D = D;
  a.in_f32 = x->dtype == GLA_F32;
  a.out_f32 = y->dtype == GLA_F32;
  if (gla::launch_conv_fwd(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_conv1d_step(int64_t N, int64_t D, const gla_tensor* x, const float* w, const float* bias,
                           float* state, int64_t state_stride_n, gla_tensor* y, void* stream) {
  if (!x || !w || !state || !y) return GLA_ERR_NULL;
  if (N < 1 || !conv_dims_ok(D) || N > ((int64_t)1 << 30)) return GLA_ERR_SHAPE;
  if (gla::conv_step_blocks(N, D) > (int64_t)0xFFFFFFFF / gla::conv_block_threads()) return GLA_ERR_SHAPE;
  if (state_stride_n < (GLA_CONV_WIDTH - 1) * D) return GLA_ERR_SHAPE;
  gla_status st;
  if ((st = check_act(x, N, 1, D)) != GLA_OK) return st;
  if ((st = check_act(y, N, 1, D)) != GLA_OK) return st;
  if (!aligned16(w) || !aligned16(bias) || !aligned16(state) || (N > 1 && (state_stride_n * 4) % 16 != 0))
    return GLA_ERR_STRIDE;
  const void* ins[] = {x->data, w, bias};
  for (const void* p : ins)
    if (same(y->data, p) || same(state, p)) return GLA_ERR_ALIAS;
  if (same(y->data, state)) return GLA_ERR_ALIAS;

  gla::ConvStepArgs a{};
  a.x = x->data; a.sx_n = x->stride_b;
  a.w = w; a.bias = bias;
  a.state = state; a.state_stride_n = state_stride_n;
  a.y = y->data; a.sy_n = y->stride_b;
  a.N = N; a.D = D;
  a.in_f32 = x->dtype == GLA_F32;
  a.out_f32 = y->dtype == GLA_F32;
  if (gla::launch_conv_step(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

}  // extern "C"

namespace {

gla_status chunk_fwd_impl(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                          const gla_tensor* v, const float* lambda, const float* S0, gla_tensor* o,
                          float* S_T, void* ws, size_t ws_bytes, bool noalloc, void* stream) {
  if (!dims || !q || !k || !v || !o || !lambda) return GLA_ERR_NULL;
  gla_status st = check_dims(dims);
  if (st != GLA_OK) return st;
  const int64_t B = dims->B, H = dims->H, T = dims->T;
  if (!dtype_ok(q->dtype) || !dtype_ok(o->dtype) || k->dtype != q->dtype || v->dtype != q->dtype)
    return GLA_ERR_DTYPE;
  const int in_f32 = q->dtype == GLA_F32;
  if (!gla::chunk_pass_supported((int)dims->dk, (int)dims->dv, (int)dims->chunk, in_f32))
    return GLA_ERR_UNSUPPORTED;
  const bool need = T > 0;
  const int64_t DK = dims->dk, DV = dims->dv, C = dims->chunk;
  if ((st = check_view(q, B, H, T, DK, C, need)) != GLA_OK) return st;
  if ((st = check_view(k, B, H, T, DK, C, need)) != GLA_OK) return st;
  if ((st = check_view(v, B, H, T, DV, C, need)) != GLA_OK) return st;
  if ((st = check_view(o, B, H, T, DV, C, need)) != GLA_OK) return st;
  if (!aligned16(S0) || !aligned16(S_T) || !aligned16(lambda)) return GLA_ERR_STRIDE;
  if (same(o->data, q->data) || same(o->data, k->data) || same(o->data, v->data) ||
      same(S_T, S0) || same(S_T, q->data) || same(S_T, k->data) || same(S_T, v->data) ||
      same(S_T, o->data) || same(S_T, lambda) || same(o->data, lambda) || same(o->data, S0))
    return GLA_ERR_ALIAS;
  const size_t need_ws = gla_chunk_fwd_workspace(dims);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (noalloc) {
    // the segment states must fit the static scratch; nothing in it needs to
    // start at zero (the state pass writes every entry the full pass reads)
    if (need_ws > GLA_NOALLOC_SCRATCH_BYTES) return GLA_ERR_WORKSPACE;
    ws = nullptr;
    if (need_ws > 0 && (st = noalloc_scratch(s, &ws)) != GLA_OK) return st;
  } else if (ws_bytes < need_ws || (need_ws > 0 && (ws == nullptr || !aligned16(ws)))) {
    return GLA_ERR_WORKSPACE;
  }

  ChunkArgs a = make_pass(dims, q, k, v, lambda, S0, 0, S_T, o, 0);
  set_segments_flags(a, dims, (int)dims->dk, (int)dims->dv, ws);
  if (gla::launch_chunk_pass((int)dims->dk, (int)dims->dv, (int)dims->chunk, a, s) != hipSuccess)
    return GLA_ERR_HIP;
  return GLA_OK;
}

}  // namespace
