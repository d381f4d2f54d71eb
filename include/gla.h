/*
 * gla.h -- C ABI of the Simple GLA mixer library (libgla.so, AMD MI355X /
 * gfx950).
 *
 * The operation is the token mixer described on the page "Beyond the KV
 * cache: Training and serving i14's Laplace 3B linear attention model on AWS
 * Trainium2 with native PyTorch":
 *   - section "GLA mixer": every head h keeps a dk x dv matrix state that is
 *     decayed by a fixed per-head factor lambda_h and receives the rank-1
 *     write of the current key/value pair; the output queries the state:
 *         S_t = lambda_h * S_{t-1} + k_t v_t^T,     o_t = S_t^T q_t
 *     (the readout sees the updated state, so o_t includes token t itself);
 *   - section "Challenge 1": the chunked form used for prefill and training
 *     (masked linear attention inside each chunk plus the running state; the
 *     state advances by the decay compounded over the chunk);
 *   - section "Challenge 3": the backward pass through the sequential state
 *     updates;
 *   - sections "GLA mixer" and "Inference optimization on Trainium2": the
 *     O(1)-per-token recurrent decode step against a fixed-size state.
 *
 * Conventions shared by every entry point
 *   Ownership   The caller owns every buffer.  Pointers are HIP device
 *               pointers unless stated otherwise.  The library never
 *               allocates or frees; transient memory comes from the caller's
 *               workspace, sized by the matching *_workspace() query.
 *   Streams     `stream` is a hipStream_t passed as void* (NULL = the null
 *               stream).  Every call only enqueues work and returns without
 *               synchronising; buffers must stay valid until it completes.
 *   Errors      All arguments are validated on the host before anything is
 *               enqueued; on a non-OK status nothing was enqueued.  A launch
 *               failure returns GLA_ERR_HIP.  Faults inside kernels surface at
 *               the caller's next synchronisation.  No C++ exception crosses
 *               the ABI.  Calls keep no global state and are thread-safe,
 *               except gla_chunk_fwd_noalloc, whose device scratch is
 *               shared by every call on one GPU.
 *   Tensors     gla_tensor describes a 4-D (b, h, t, d) view: element
 *               (b, h, t, d) lives at data + (b*stride_b + h*stride_h +
 *               t*stride_t + d) elements; d is contiguous.  Strides are in
 *               elements, non-negative.  The base pointer and every row start
 *               must be 16-byte aligned; rows along t must not overlap
 *               (stride_t >= d) and stride_t * element size * chunk must be
 *               below 2^31 bytes (GLA_ERR_STRIDE otherwise).  Both the
 *               head-major [B,H,T,d] and the token-major [B,T,H,d] layouts
 *               are accepted without copies.
 *   Dtypes      q, k, v (and dO) share one dtype, GLA_BF16 or GLA_F32.
 *               Outputs o, dq, dk, dv may each be GLA_BF16 or GLA_F32.  All
 *               states (S0, S_T, dS_T, dS0, decode S) and lambda are fp32,
 *               dense row-major [B][H][dk][dv] (dk rows of dv).
 *   Shapes      (dk, dv) in {(96, 192), (16, 32)}; chunk in {16, 32, 64, 128}.
 *               fp32 inputs need chunk <= 64, and chunk <= 32 for the
 *               backward at (96, 192).  Other combinations return
 *               GLA_ERR_UNSUPPORTED.  B, H >= 1; T >= 0 (T = 0 copies the
 *               state through); T need not be a multiple of chunk.
 *               B <= 2^24, H <= 2^16, B * H <= 2^21 and T <= 2^40
 *               (GLA_ERR_SHAPE otherwise): one launch addresses at most
 *               2^32 - 1 work-items.
 *   Chunk       the tile length of the chunked form.  Results are equal up
 *               to rounding for every chunk: the chunked form computes the
 *               recurrence's sums exactly, and only the order of its
 *               floating-point additions depends on the chunk.  Every
 *               pass tiles at the chunk, except that at chunk 128 with bf16
 *               inputs the backward's dq and dk passes (a 192 x 96 state)
 *               tile at 64 tokens, their 128-token tiles fitting no layout
 *               of more than three waves per compute unit, and so does
 *               gla_chunk_fwd_fused (its output staging does not fit).
 *   Decay       lambda[h] must satisfy 0 <= lambda[h] <= 1 (not checked on
 *               the device); 0^0 is taken as 1.  NaN/Inf inputs propagate.
 *   Aliasing    Outputs must not share a base pointer with any input or with
 *               each other (GLA_ERR_ALIAS); the decode state is in/out.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_ABI_VERSION 2

typedef enum {
  GLA_OK = 0,
  GLA_ERR_NULL = 1,        /* a required pointer is NULL */
  GLA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  GLA_ERR_STRIDE = 3,      /* negative stride or a misaligned row start */
  GLA_ERR_DTYPE = 4,       /* unknown dtype or q/k/v dtypes differ */
  GLA_ERR_UNSUPPORTED = 5, /* (dk, dv, chunk, dtype) has no compiled kernel */
  GLA_ERR_ALIAS = 6,       /* an output aliases an input or another output */
  GLA_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required */
  GLA_ERR_HIP = 8          /* the HIP runtime reported a launch error */
} gla_status;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;

typedef struct {
  void* data;
  int32_t dtype; /* gla_dtype */
  int64_t stride_b, stride_h, stride_t;
} gla_tensor;

typedef struct {
  int64_t B, H, T, dk, dv, chunk;
} gla_dims;

/* ABI version of the loaded library (GLA_ABI_VERSION). */
int gla_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* gla_status_string(gla_status s);

/* Bytes of device workspace gla_chunk_fwd needs for these dims (0 if none).
 * Returns 0 for dims that gla_chunk_fwd would reject.
 * When B * H is too small to occupy the GPU, a pass splits every sequence
 * into nseg segments of whole chunks (2 <= nseg <= 64, at least two chunks
 * each; page section "Challenge 1": the chunks are independent apart from the
 * state they hand on).  Each segment's end state from a zero start is written
 * to the workspace, and segment j starts from the decayed sum of the end
 * states before it.  When the split's workgroups fit the device's compute
 * units one each, both happen in one launch: a workgroup publishes its
 * segment's end state with an 8-byte flag and reads the earlier ones once
 * their flags are set (otherwise two launches).  The workspace holds
 * B*H*nseg*dk*dv fp32 states followed by B*H*nseg*ceil(dv/16) flags, rounded
 * up to 16 bytes; ws must be 16-byte aligned
 * (GLA_ERR_WORKSPACE otherwise).  Nothing in it needs to start at zero (a
 * flag counts only if it carries the call's own tag) and its contents are
 * not needed after the call completes. */
size_t gla_chunk_fwd_workspace(const gla_dims* dims);

/* Tuning of the one-launch segment split (gla_chunk_fwd, gla_chunk_bwd,
 * gla_chunk_fwd_noalloc): how long, in
 * microseconds, a workgroup waits for an earlier segment's end state before
 * forming that state itself (by the same arithmetic, so results never
 * depend on it).  Negative restores the default, about four times a
 * segment's state pass; 0 forms at once every state not yet published.
 * Process-wide; takes effect for calls made after it. */
void gla_set_segment_wait(int32_t microseconds);

/* Chunked forward (page sections "GLA mixer" and "Challenge 1").
 *   q [B,H,T,dk], k [B,H,T,dk], v [B,H,T,dv]   inputs (gla_tensor views)
 *   lambda [H] fp32                            per-head decay
 *   S0 [B,H,dk,dv] fp32 or NULL                state before token 1 (NULL = 0)
 *   o [B,H,T,dv]                               output (bf16 or fp32)
 *   S_T [B,H,dk,dv] fp32 or NULL               state after token T
 *   ws, ws_bytes                               workspace (may be NULL if the
 *                                              query returned 0)
 * o_t = lambda^t S0^T q_t + sum_{s<=t} lambda^{t-s} (q_t . k_s) v_s. */
gla_status gla_chunk_fwd(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                         const gla_tensor* v, const float* lambda, const float* S0,
                         gla_tensor* o, float* S_T, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch that gla_chunk_fwd_noalloc uses in
 * place of a workspace (16 MiB per GPU). */
#define GLA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* gla_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as gla_chunk_fwd, without ws/ws_bytes:
 * the segment states go to a library-owned static array of
 * GLA_NOALLOC_SCRATCH_BYTES on the device that runs `stream` (each GPU keeps
 * its copy until the process ends; its address is looked up once per device
 * on the first call there).  The call allocates nothing: it makes no
 * hipMalloc/hipFree or allocating library call.
 *   Limit   dims whose gla_chunk_fwd_workspace() exceeds the scratch return
 *           GLA_ERR_WORKSPACE before anything is enqueued; at dk=96, dv=192
 *           that is B*H in 114..127 with T of at least 4 chunks (254 segment
 *           states of 73,728 bytes, with 96 bytes of flags each, at most,
 *           against 227 that fit).
 *   Sharing Every call on one GPU uses the same scratch: calls that overlap
 *           on that GPU (different streams or host threads without ordering)
 *           race and must be serialised by the caller.  Calls ordered on one
 *           stream are safe; nothing in the scratch needs to start at zero,
 *           since each call writes every entry before reading it. */
gla_status gla_chunk_fwd_noalloc(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                                 const gla_tensor* v, const float* lambda, const float* S0,
                                 gla_tensor* o, float* S_T, void* stream);

/* Bytes of device workspace gla_chunk_bwd needs (0 if none): the segment
 * states and flags (as for gla_chunk_fwd_workspace) of its paired dq/dk
 * passes, two regions, or of its dv pass, whichever is larger (the dv pass
 * reuses the space); the dq/dk passes' segments follow their own tile length
 * (see Chunk above).  Nothing in it needs to start at zero. */
size_t gla_chunk_bwd_workspace(const gla_dims* dims);

/* Chunked backward (page section "Challenge 3") of the scalar
 *   L = sum_t <dO_t, o_t> + <dS_T, S_T>
 * with o, S_T the forward outputs for the same (q, k, v, lambda, S0):
 *   dO [B,H,T,dv]       upstream gradient of o (same dtype as q, k, v)
 *   dS_T fp32 or NULL   upstream gradient of S_T (NULL = 0)
 *   dq [B,H,T,dk], dk [B,H,T,dk], dv [B,H,T,dv]  outputs (bf16 or fp32)
 *   dS0 [B,H,dk,dv] fp32 or NULL                 gradient of S0 (NULL = skip)
 * lambda is fixed (not learned), so there is no gradient for it. */
gla_status gla_chunk_bwd(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                         const gla_tensor* v, const float* lambda, const float* S0,
                         const gla_tensor* dO, const float* dS_T, gla_tensor* dq,
                         gla_tensor* dk, gla_tensor* dv, float* dS0, void* ws,
                         size_t ws_bytes, void* stream);

/* One recurrent decode step for N sequences x H heads (page sections "GLA
 * mixer" and "Inference optimization on Trainium2"):
 *   S <- lambda S + k v^T (in place),  then  o = S^T q.
 *   q, k [N,H,dk]; v, o [N,H,dv]  gla_tensor views with stride_b = stride
 *                                 over n, stride_h over h (stride_t unused)
 *   S    fp32, sequence n / head h at S + n*S_stride_n + h*dk*dv, dense
 *        dk x dv per head; S_stride_n >= H*dk*dv elements (a per-sequence
 *        page may hold further layers' states), 16-byte aligned.
 *   N, H >= 1, N * H <= 2^24 (GLA_ERR_SHAPE otherwise). */
gla_status gla_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, const gla_tensor* q,
                           const gla_tensor* k, const gla_tensor* v, const float* lambda,
                           float* S, int64_t S_stride_n, gla_tensor* o, void* stream);

/* Launch shape of the decode step, for capacity planning and tests (calling
 * it is never required): the number of workgroups gla_decode_step (fused =
 * 0), gla_decode_step_fused with its workspace (fused = 1) or without one
 * (fused = 2) launches per (n, h) state for these sizes, or 0 when that call
 * would reject them (or fused is outside 0..2).  At (96, 192) the plain step
 * and the fused step with its workspace split each state into 3 column
 * slices while N * H * 3 * 384 work-items fit one launch (up to 3,728,270
 * states), else they run one workgroup per state; the fused step without a
 * workspace always runs one workgroup per state. */
int gla_decode_workgroups_per_state(int64_t N, int64_t H, int64_t dk, int64_t dv, int fused);

/* Chunked forward with the mixer's output epilogue fused into the store
 * (page section "GLA mixer", after the readout: self-augmentation adds a
 * gated copy of the value, the gate being the sigmoid of the query-key dot
 * product with a learned per-channel scale a, zero at initialisation; each
 * head's output then goes through the Head RMSNorm of its decay tier and is
 * gated by SiLU(g_t) before the output projection).  Per token and head:
 *   o' = o + sigmoid(sum_i q[i] aug[h][i] k[i]) v
 *   y  = o' / sqrt(mean_j o'[j]^2 + eps) * gamma[h] * SiLU(g)
 * with o the output of gla_chunk_fwd; y replaces o.
 *   g      the gate stream [B,H,T,dv] (same dtype and view rules as q, k, v;
 *          the model's token-major [B, T, H*dv] layout is the view with
 *          stride_h = dv, stride_t = H*dv)
 *   aug    fp32 [H][dk];  gamma fp32 [H][dv] (a tier's RMSNorm weight,
 *          repeated for each head of the tier);  eps >= 0 (GLA_ERR_SHAPE
 *          otherwise)
 * Shapes: (dk, dv) in {(96, 192), (16, 32)}; chunk in {16, 32, 64, 128}
 * (fp32 inputs: 16 or 32 at (96, 192), up to 64 at (16, 32)).  With bf16
 * inputs chunk 128 tiles at 64 tokens: a 128-token tile's fp32 output
 * staging does not fit beside its tiles (results are equal up to rounding,
 * see Chunk above).  Workspace from gla_chunk_fwd_fused_workspace (segment
 * states, as for gla_chunk_fwd). */
size_t gla_chunk_fwd_fused_workspace(const gla_dims* dims);
gla_status gla_chunk_fwd_fused(const gla_dims* dims, const gla_tensor* q, const gla_tensor* k,
                               const gla_tensor* v, const float* lambda, const float* S0,
                               const gla_tensor* g, const float* aug, const float* gamma, float eps,
                               gla_tensor* y, float* S_T, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace gla_decode_step_fused can use for these sizes
 * (0 when the step runs one workgroup per state anyway, or the sizes are
 * rejected): N*H*(dv + 4) fp32 values at (96, 192). */
size_t gla_decode_step_fused_workspace(int64_t N, int64_t H, int64_t dk, int64_t dv);

/* gla_decode_step with the same output epilogue as gla_chunk_fwd_fused
 * applied to o before it is written (y replaces o):
 *   g      the gate stream [N, H, dv] view (stride_b steps n, stride_h h;
 *          same dtype as q, k, v)
 *   aug    fp32 [H][dk]; gamma fp32 [H][dv]; eps >= 0
 *   ws, ws_bytes  optional workspace of gla_decode_step_fused_workspace()
 *          bytes, 16-byte aligned, not shared with any other argument
 *          (GLA_ERR_WORKSPACE / GLA_ERR_ALIAS otherwise).  With it, the step
 *          streams each state as column slices and normalises in a second
 *          kernel (faster); with ws = NULL one workgroup owns each state and
 *          normalises its row itself.  Both give the same state; outputs
 *          agree up to the summation order of the sum of squares.  The
 *          workspace is scratch, not needed after the call completes. */
gla_status gla_decode_step_fused(int64_t N, int64_t H, int64_t dk, int64_t dv, const gla_tensor* q,
                                 const gla_tensor* k, const gla_tensor* v, const float* lambda, float* S,
                                 int64_t S_stride_n, const gla_tensor* g, const float* aug,
                                 const float* gamma, float eps, gla_tensor* y, void* ws, size_t ws_bytes,
                                 void* stream);

/* Variable-length batched prefill straight into the decode state pool (page
 * sections "GLA mixer" and "Inference optimization on Trainium2": each
 * sequence owns one fixed-size state page that prefill fills and every decode
 * step then reads and writes).  N packed sequences, the forward of
 * gla_chunk_fwd per sequence and head:
 *   q, k [total_T, H, dk]; v, o [total_T, H, dv]  packed gla_tensor views:
 *          element (t, h, d) at data + t*stride_t + h*stride_h + d
 *          (stride_b unused); same dtype and layout rules as gla_chunk_fwd
 *   cu_seqlens  device int32 [N+1]: sequence n is tokens [cu[n], cu[n+1]).
 *          Entries are clamped to [0, total_T] and made non-decreasing on the
 *          device, so bad offsets cannot reach outside the packed tensors.
 *   pool   fp32 pages: sequence n's state for head h is the dense dk x dv
 *          block at pool + slot*pool_stride_n + h*dk*dv, slot = slots[n]
 *          (device int32 [N], or n when slots is NULL); pool_stride_n >=
 *          H*dk*dv (a page may hold further layers), a multiple of 4 when
 *          num_slots > 1.  Sequences whose slot is outside [0, num_slots)
 *          are skipped (nothing read or written for them).
 *   has_state  device int32 [N] or NULL: the sequence starts from its page's
 *          state when nonzero (NULL: every sequence does), else from zero.
 *   N, H >= 1, N * H <= 2^21, total_T < 2^31 (GLA_ERR_SHAPE otherwise).
 *          The final state is written back to the page (in place).
 * No workspace.  Slots must be distinct (two sequences writing one page
 * race). */
gla_status gla_chunk_fwd_varlen(int64_t N, int64_t H, int64_t total_T, int64_t dk, int64_t dv,
                                int64_t chunk, const gla_tensor* q, const gla_tensor* k,
                                const gla_tensor* v, const int32_t* cu_seqlens, const float* lambda,
                                float* pool, int64_t num_slots, int64_t pool_stride_n,
                                const int32_t* slots, const int32_t* has_state, gla_tensor* o,
                                void* stream);

/* ------------------------------------------------------------------------
 * Depthwise causal convolution (width GLA_CONV_WIDTH) + SiLU, the step in
 * front of the mixer (page section "i14 and Laplace 3B architecture",
 * paragraph "Normalization and convolution": every channel of the
 * D = 3,072-wide residual stream is convolved causally over its last 4
 * tokens and passed through SiLU; the window belongs to the per-sequence
 * recurrent state).  For token t and channel c:
 *   z = bias[c] + sum_{j<4} w[c][j] * x[t-3+j][c],   y[t][c] = z / (1 + exp(-z))
 * so w[c][3] weights the current token.  Inputs before token 0 come from the
 * carried window (oldest first), zero when it is NULL.  Arithmetic is fp32.
 *   x, y      gla_tensor views of [B, T, D]: element (b, t, c) at
 *             data + b*stride_b + t*stride_t + c (stride_h unused); bf16 or
 *             fp32 each; 16-byte aligned rows, stride_t >= D
 *   D         multiple of 8, 8 <= D <= 2^24; a call's launch must stay below
 *             2^32 work-items (one per 8 channels of 16 tokens, or of one
 *             token in the decode step; GLA_ERR_SHAPE otherwise)
 *   w         fp32 [D][4];  bias fp32 [D] or NULL
 *   windows   fp32 [B][3][D], 16-byte aligned
 * ------------------------------------------------------------------------ */
#define GLA_CONV_WIDTH 4

/* Prefill / training forward over T tokens (T = 0 copies state_in, or zeros,
 * to state_out).  state_out (the last 3 inputs, ready for decode) may be
 * NULL; it must not alias state_in. */
gla_status gla_conv1d_fwd(int64_t B, int64_t T, int64_t D, const gla_tensor* x, const float* w,
                          const float* bias, const float* state_in, gla_tensor* y, float* state_out,
                          void* stream);

/* One decode token for N sequences: y = SiLU(bias + w . [window, x]), then
 * the window drops its oldest input and appends x, in place.
 *   x, y   [N, D] views (stride_b steps n; stride_t unused)
 *   state  sequence n's window at state + n*state_stride_n, [3][D] fp32;
 *          state_stride_n >= 3*D (a per-sequence page may hold further
 *          layers), a multiple of 4 when N > 1. */
gla_status gla_conv1d_step(int64_t N, int64_t D, const gla_tensor* x, const float* w, const float* bias,
                           float* state, int64_t state_stride_n, gla_tensor* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
