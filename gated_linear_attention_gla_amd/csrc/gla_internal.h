// gla_internal.h -- argument blocks and launcher declarations shared between
// the host library (gla_api.cpp) and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

// One pass of the generic chunked recurrence over "roles" (qr, kr, vr):
//   state  S (DK x DV, fp32, per (b, h)), decay lam[h]
//   forward time:  S_t = lam S_{t-1} + kr_t vr_t^T,  out_t = S_t^T qr_t
//   reverse time:  the same recurrence run from the last token to the first.
// The chunked forward uses (q, k, v); the backward runs three passes with the
// roles permuted (see gla_api.cpp).
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t sq_b, sq_h, sq_t;  // element strides of the query role
  int64_t sk_b, sk_h, sk_t;
  int64_t sv_b, sv_h, sv_t;
  void* o;
  int64_t so_b, so_h, so_t;
  const float* lam;       // [H]
  const float* s_init;    // [B][H] x (DK x DV) or null (zero state)
  int s_init_trans;       // 1: element (d, n) stored at n * DK + d
  float* s_final;         // [B][H][DK][DV] or null
  int64_t B, H, T;
  int reverse;            // 0: tokens 0..T-1, 1: tokens T-1..0
  int o_f32;              // output storage: 1 fp32, 0 bf16
  int in_f32;             // input storage:  1 fp32, 0 bf16 (must match the instantiation)
  // Segment-parallel form: tokens split into nseg segments of seg_len tokens
  // (a multiple of the chunk; the last may be shorter).  seg_state holds,
  // per (b, h) and segment, the segment's end state from a zero start
  // ([B][H][nseg] x (DK x DV), fp32); the state pass writes it and the full
  // pass folds the earlier segments' states into its entry state.
  int nseg;
  int64_t seg_len;
  float* seg_state;
  // One-launch split (seg_flag set): every workgroup runs its own segment's
  // state pass, publishes it with its flag (index (bh NBLK + column block)
  // nseg + segment) set to seg_tag | the XCD it ran on, and folds an earlier
  // segment's state once that flag reads the same tag and XCD (same L2);
  // after seg_wait ticks of the 100 MHz clock it forms the state itself.
  // Each workgroup clears its flag on exit.
  unsigned long long* seg_flag;
  unsigned long long seg_tag;  // per-call nonzero epoch << 8
  uint32_t seg_wait;
  // Packed variable-length mode (prefill into the decode state pool).  With
  // cu set, unit b covers tokens [cu[b], cu[b+1]) of the packed inputs
  // (clamped to [0, T]; stride_b is then 0).  With pool set, unit (b, h)
  // keeps its state in page slots[b] (or b) of the pool, at
  // pool + slot * pool_stride_n + h * DK * DV: read at the start unless
  // has_state[b] == 0, written back at the end; a slot outside
  // [0, num_slots) skips the unit.  Neither mode splits segments.
  const int32_t* cu;
  float* pool;
  int64_t pool_stride_n, num_slots;
  const int32_t* slots;
  const int32_t* has_state;
  // Output epilogue (forward with every column of a head in one workgroup):
  // o' = o + sigmoid(q . (aug_h * k)) v, y = o' / sqrt(mean(o'^2) + eps) *
  // gamma_h * SiLU(gz), written to o.  gz: the gate stream, (b, h, t, d)
  // strides like the other inputs and in their dtype.
  const void* gz;
  int64_t sg_b, sg_h, sg_t;
  const float* aug;    // [H][DK]
  const float* gamma;  // [H][DV]
  float eps;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t sq_n, sq_h, sk_n, sk_h, sv_n, sv_h;
  const float* lam;
  float* S;
  int64_t S_stride_n;  // elements between consecutive sequences; heads are dense
  void* o;
  int64_t so_n, so_h;
  int64_t N, H;
  int o_f32;
  int in_f32;
  // output epilogue (the fused decode step): gate stream g [N, H, dv] view,
  // aug [H][DK], gamma [H][DV], eps; null gz = plain step
  const void* gz;
  int64_t sg_n, sg_h;
  const float* aug;
  const float* gamma;
  float eps;
  // fused step's workspace (split epilogue), or null: o' [N*H][DV] fp32, then
  // the column slices' sums of squares [N*H][4]
  float* ws;
};

// Depthwise causal convolution (width 4) + SiLU over [B][T][D] activations.
struct ConvArgs {
  const void* x;
  int64_t sx_b, sx_t;      // element strides of x (channels contiguous)
  const float* w;          // [D][4]
  const float* bias;       // [D] or null
  const float* state_in;   // [B][3][D] inputs before token 0, or null (zeros)
  void* y;
  int64_t sy_b, sy_t;
  float* state_out;        // [B][3][D] last 3 inputs, or null
  int64_t B, T, D;
  int in_f32, out_f32;
};

// One decode token per sequence; the window is updated in place.
struct ConvStepArgs {
  const void* x;
  int64_t sx_n;
  const float* w;
  const float* bias;
  float* state;            // sequence n at state + n * state_stride_n, [3][D]
  int64_t state_stride_n;
  void* y;
  int64_t sy_n;
  int64_t N, D;
  int in_f32, out_f32;
};

// Launchers return hipSuccess or the launch error.  They perform no
// validation: the C-ABI layer checks every argument first.
// One chunked pass; with a.nseg > 1 this is the segment state pass followed
// by the full pass.
hipError_t launch_chunk_pass(int dk, int dv, int chunk, const ChunkArgs& a, hipStream_t st);
// Two passes of a shape with dk > dv in one launch: a0 in forward time, a1 in
// reverse time, same B, H, T and segments (each with its own seg_state).
hipError_t launch_chunk_pair(int dk, int dv, int chunk, const ChunkArgs& a0, const ChunkArgs& a1,
                             hipStream_t st);
// Segments used for these dims (1 = no segment split) and the workspace bytes
// they need: enough (b, h, column block, segment) units to fill the GPU.
int chunk_segments(int64_t B, int64_t H, int64_t T, int dk, int dv, int chunk, int in_f32);
bool chunk_pass_supported(int dk, int dv, int chunk, int in_f32);
int bwd_transposed_tile(int chunk, int in_f32);
// Segments for a given number of (b, h, column block) units.
int segments_for_units(int64_t units, int64_t T, int chunk);
// Forward with the fused output epilogue (whole heads per workgroup).
bool chunk_fused_supported(int dk, int dv, int chunk, int in_f32);
int chunk_segments_fused(int64_t B, int64_t H, int64_t T, int chunk);
int fused_tile(int chunk, int in_f32);
hipError_t launch_chunk_fused(int dk, int dv, int chunk, const ChunkArgs& a, hipStream_t st);
hipError_t launch_decode(int dk, int dv, const DecodeArgs& a, hipStream_t st);
bool decode_supported(int dk, int dv);
// Workgroups (column slices) the decode step launches per state for `states`
// states (0 when the shape has no kernel), plain or fused (epi), the fused
// step with or without its workspace; the launch stays below 2^32 work-items
// for every state count the ABI accepts.
int decode_slices(int64_t states, int dk, int dv, bool epi, bool has_ws);
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st);
hipError_t launch_conv_step(const ConvStepArgs& a, hipStream_t st);
// one-dimensional grid sizes of the two convolution launches, and their
// workgroup sizes (decode step, prefill)
int64_t conv_fwd_blocks(int64_t B, int64_t T, int64_t D);
int64_t conv_step_blocks(int64_t N, int64_t D);
int conv_block_threads();
int conv_fwd_threads();

}  // namespace gla
