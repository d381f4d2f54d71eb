// gla_chunk.hip -- chunked Simple GLA recurrence on CDNA4 bf16 MFMA.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Challenge 1"
// (inside a chunk the output is decay-masked linear attention plus the
// running state's contribution; the state then advances by the decay
// compounded over the chunk, and only that advance is sequential) and section
// "GLA mixer" (S_t = lam S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, per head).
//
// For a chunk of L tokens with local index i, j in [0, L) and state S on
// entry, in forward time:
//   O[i]  = lam^{i+1} (S^T q_i) + sum_{j<=i} lam^{i-j} (q_i . k_j) v_j
//   S    <- lam^L S + sum_j lam^{L-1-j} k_j v_j^T
// In reverse time (used by the backward) the window is j >= i, the mask is
// lam^{j-i}, the state enters with lam^{L-1-i} and advances with lam^{j+1}.
// Only non-negative powers lam^n, n <= chunk, are ever formed (fp32 table).
//
// One workgroup owns one (b, h) and a BN-wide block of state/output columns
// and walks the chunks in order, keeping its DK x BN slice of the fp32 state
// in MFMA accumulators.  Each wave owns NS strips of 16 columns.  Per chunk:
//   stage 0  q, k, v tiles -> LDS (bf16 planes; fp32 inputs become 3 planes)
//   stage 1  P^T = K Q^T tiles (causal half only), masked in fp32 -> LDS
//   stage 2  O^T = S^T Q^T, scaled by the row factors (state split hi+lo)
//   stage 3  O^T += V^T P^T, store O (O^T tiles give each lane 4 adjacent columns)
//   stage 4  S = lam^L S + K^T (col factors * V)  (scaled V split hi+lo)
// Operands that are not exact bf16 values (the masked P tile, the state, the
// decay-scaled values) enter the MFMA as hi+lo bf16 pairs (three terms for fp32
// inputs), which keeps every product at fp32-level accuracy.
#include <atomic>
#include <type_traits>

#include "gla_common.hpp"
#include "gla_internal.h"

// cache policy of a buffer access: sc1 (device scope)
constexpr int kCpolSc1 = 16;

namespace gla {

// sigmoid(x) = 1 / (1 + e^-x) from the hardware base-2 exponential and reciprocal (each
// within about one ulp; the product x log2(e) adds |x| 2^-24 to the
// exponent), a relative error near 1e-6 for |x| < 10.  Large negative x
// gives 1 / inf = 0, large positive x gives 1.
__device__ __forceinline__ float sigmoid_hw(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// lam^n for n >= 0 in fp32, computed in double; 0^0 = 1.
__device__ __forceinline__ float lam_pow_f32(float lam, int n) {
  if (n == 0) return 1.0f;
  if (lam == 0.0f) return 0.0f;
  if (lam == 1.0f) return 1.0f;
  return (float)exp2((double)n * log2((double)lam));
}

template <int NT>
__device__ __forceinline__ void store_planes8(bf16_t* dst0, int plane_stride, const float (&x)[8]) {
  // x -> NT bf16 planes, 16 bytes per plane
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 t[NT];
      split_terms<NT>(x[e], t);
      v[e] = t[p];
    }
    *reinterpret_cast<bf16x8*>(dst0 + (size_t)p * plane_stride) = v;
  }
}

// Raw storage of 8 consecutive input elements held in registers between the
// global load and the LDS store: one 16-byte vector for bf16 inputs, two for
// fp32 inputs (only the NT == 3 instantiations read fp32).
template <int NT> struct Raw8;
template <> struct Raw8<1> { bf16x8 v; };
template <> struct Raw8<3> { f32x4 a, b; };

// A (ROWS x COLS) tile of one chunk, staged global -> registers -> LDS.
// Thread tid owns the 8-element vectors tid, tid + NTHR, ...; since NTHR is a
// multiple of the vectors per row, its column is fixed and its rows step by
// RPJ.  Loads go through a buffer resource whose size ends at the last valid
// row, so rows >= L read as zero without branches; columns in [COLS, COLSP)
// are zero.  LDS holds NT bf16 planes with row pitch PITCH.  With SWZ, rows
// whose bit 3 is set hold their 16-column groups pairwise exchanged (column c
// at c ^ 16), the layout the readers of such tiles assume (tile_swz).
template <int NT, int ROWS, int COLS, int COLSP, int PITCH, int NTHR, bool SWZ = false>
struct TileStager {
  static constexpr int VPR = COLSP / 8;
  static_assert(NTHR % VPR == 0, "threads must cover whole rows");
  static constexpr int RPJ = NTHR / VPR;  // rows advanced per step j
  static constexpr int NPER = (ROWS + RPJ - 1) / RPJ;
  static constexpr int PLANE = ROWS * PITCH;
  static constexpr int ES = NT == 1 ? 2 : 4;  // input element size
  static_assert(!SWZ || COLSP % 32 == 0, "the swizzle exchanges 16-column groups within 32");
  Raw8<NT> r[NPER];

  // gsrc: the tile's first row; row_stride in elements; L valid rows (>= 1)
  __device__ __forceinline__ void load(const void* gsrc, uint32_t row_stride, int L, int tid) {
    const int row0 = tid / VPR;
    const int c = (tid - row0 * VPR) * 8;
    const uint32_t nbytes = ((uint32_t)(L - 1) * row_stride + COLS) * ES;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(gsrc), (short)0, (int)nbytes, 0x00020000);
    const uint32_t voff = ((uint32_t)row0 * row_stride + c) * ES;
    const uint32_t jstep = (uint32_t)RPJ * row_stride * ES;
    const bool col_ok = COLSP == COLS || c < COLS;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      if constexpr (NT == 1) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
        if (col_ok) v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * jstep, 0));
        r[j].v = v;
      } else {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (col_ok) {
          x0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * jstep, 0));
          x1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, j * jstep, 0));
        }
        r[j].a = x0;
        r[j].b = x1;
      }
    }
  }

  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    const int row0 = tid / VPR;
    const int c = (tid - row0 * VPR) * 8;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int row = row0 + j * RPJ;
      if (ROWS % RPJ == 0 || row < ROWS) {
        bf16_t* dst = lds + row * PITCH + (SWZ ? c ^ ((row & 8) << 1) : c);
        if constexpr (NT == 1) {
          *reinterpret_cast<bf16x8*>(dst) = r[j].v;
        } else {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = r[j].a[e];
            x[4 + e] = r[j].b[e];
          }
          store_planes8<NT>(dst, PLANE, x);
        }
      }
    }
  }
};

// Causal P tiles in the forward enumeration: t -> (I', J') with J' <= I',
// t = I'(I'+1)/2 + J'.  Wave-uniform, branch-free scalar arithmetic.
template <int CT>
__device__ __forceinline__ void tile_of(int t, int& Ip, int& Jp) {
  int i = 0;
#pragma unroll
  for (int m = 1; m < CT; ++m) i += (t >= m * (m + 1) / 2) ? 1 : 0;
  Ip = i;
  Jp = t - i * (i + 1) / 2;
}

// P-tile row pitch: the smallest >= CP + 8 (multiple of 8 elements) whose
// byte pitch mod 256 is 32, 160 or 224 -- conflict-free 16-byte row reads.
constexpr int pitch_p(int cp) {
  for (int p = cp + 8;; p += 8) {
    const int m = (2 * p) % 256;
    if (m == 32 || m == 160 || m == 224) return p;
  }
}

// Key-tile row pitch: the smallest >= DKP (multiple of 8 elements) whose byte
// pitch mod 256 is 192 -- the transposing column reads of the state update
// (16 lanes: 4 rows x 4 column groups 16 bytes apart) then cost the minimum
// 4 LDS cycles; the 16-byte row reads of the P tiles pay 4 extra cycles, but
// they are 5 times fewer.
constexpr int pitch_kt(int dkp) {
  for (int p = dkp;; p += 8)
    if ((2 * p) % 256 == 192) return p;
}

// Column swizzle of the key and value tiles (64 or more columns, a multiple of
// 32): row r keeps column c at c ^ tile_swz(r).  At a byte pitch of 192 mod
// 256, rows r and r + 8 of a transposing column read otherwise hit the same
// banks; exchanging the 16-column groups of rows with bit 3 set makes those
// reads and the 16-byte row reads of the key tile conflict-free (measured with
// rocprofv3 SQ_LDS_BANK_CONFLICT per access pattern on gfx950).  Every access
// keeps 8-element groups whole, so 16-byte stores and reads are unchanged.
constexpr bool tile_swizzled(int cols) { return cols >= 64 && cols % 32 == 0; }
__device__ __forceinline__ int tile_swz(int row) { return (row & 8) << 1; }

// State row held in accumulator slot r of row tile D by lane group g.  With DK
// a multiple of 32 the two tiles of each 32-row block interleave in runs of 4
// (tile 2m + h, group g: rows 32 m + 8 g + 4 h + r), so the 8 k-slots a lane
// group feeds to the readout are 8 consecutive state rows and the query is
// read with one 16-byte LDS read per fragment; otherwise tile D holds rows
// 16 D + 4 g + r.
template <int DK>
__device__ __forceinline__ int state_row(int D, int g, int r) {
  if constexpr (DK % 32 == 0) return 32 * (D >> 1) + 8 * g + 4 * (D & 1) + r;
  else return 16 * D + 4 * g + r;
}

// LDS layout of one chunk pass: query, key and value tiles plus the masked P
// tile (bf16 planes), the lam^n table and the per-chunk factor tables.
template <int DK, int BN, int C, int NT, int NW = 1, bool EPI = false>
struct ChunkLds {
  static constexpr int CP = (C + 31) / 32 * 32;    // chunk rows padded to the 32-deep k-step
  static constexpr int DKP = (DK + 31) / 32 * 32;  // DK padded likewise
  static constexpr int NTP = NT == 3 ? 3 : 2;      // terms of the masked P tile
  // LDS row pitches (elements), chosen from measured bank-conflict rates of
  // each tile's access mix on gfx950 (rocprofv3 SQ_LDS_BANK_CONFLICT per
  // pattern): the query and P tiles are read with 16-byte row reads
  // (conflict-free when the byte pitch mod 256 is 32, 160 or 224), the key
  // tile mostly with column reads (pitch_kt), the value tile with column reads
  // (the same cost at any pitch).
  static constexpr int PQ = DKP >= 32 ? pitch_p(DKP - 8) : DKP + 8;
  // key / value tiles swizzled (tile_swz); not at 128-token chunks or with fp32
  // inputs, where the per-lane column arithmetic would spill registers
  static constexpr bool SWK = NT == 1 && CP <= 64 && tile_swizzled(DKP);
  static constexpr bool SWV = NT == 1 && CP <= 64 && tile_swizzled(BN);
  static constexpr int PK = pitch_kt(DKP);
  static constexpr int PVV = SWV ? pitch_kt(BN) : BN + 16;
  static constexpr int PP = pitch_p(CP);
  static constexpr int Q_ELEMS = NT * CP * PQ;
  static constexpr int K_ELEMS = NT * CP * PK;
  static constexpr int V_ELEMS = NT * CP * PVV;
  static constexpr int P_ELEMS = NTP * CP * PP;
  // When the four tiles do not fit, P is held in registers until every read
  // of the query tile is done and then written over it.
  // Row-split passes (more waves than 16-column strips: RS waves share each
  // strip, each owning DK / RS state rows) sum their partial readouts
  // through an fp32 exchange tile of CP rows x BN columns.
  static constexpr int RS = NW * 16 > BN ? NW * 16 / BN : 1;
  static constexpr int XP = BN + 4;  // exchange row pitch (floats)
  static constexpr int XCH_BYTES = RS > 1 ? 4 * CP * XP : 0;
  static constexpr int SEPARATE_BYTES =
      2 * (Q_ELEMS + K_ELEMS + V_ELEMS + P_ELEMS) + 4 * (3 * CP + 2) + XCH_BYTES;
  static constexpr bool ALIAS_P = SEPARATE_BYTES > 160 * 1024 - 512;
  // output staging (see the store stage): CP rows of BN values at pitch OP2
  // (bf16) or OP4 (fp32)
  static constexpr int OP2 = BN + 8;
  static constexpr int OP4 = BN + 4;
  static constexpr int STG_ELEMS = CP * OP4 * 2;  // bf16 units, fp32 case (the larger)
  // The P region also holds the staged output when there is room for both
  // (then the next query tile can land before the output is staged, which
  // saves a barrier per chunk).
  static constexpr int P_REGION = P_ELEMS > STG_ELEMS ? P_ELEMS : STG_ELEMS;
  static constexpr bool STG_IN_P =
      !ALIAS_P && (STG_ELEMS <= P_ELEMS ||
                   2 * (Q_ELEMS + K_ELEMS + V_ELEMS + P_REGION) + 4 * (3 * CP + 2) + XCH_BYTES <=
                       160 * 1024 - 8192);
  static constexpr int QP_RAW = ALIAS_P ? (Q_ELEMS > P_ELEMS ? Q_ELEMS : P_ELEMS)
                                        : Q_ELEMS + (STG_IN_P ? P_REGION : P_ELEMS);
  static constexpr int QP_ELEMS = QP_RAW > STG_ELEMS ? QP_RAW : STG_ELEMS;
  // byte offsets (every region 16-byte aligned)
  static constexpr int OFF_K = 2 * QP_ELEMS;
  static constexpr int OFF_V = OFF_K + 2 * K_ELEMS;
  static constexpr int OFF_POW = OFF_V + 2 * V_ELEMS;
  static constexpr int OFF_ROWF = OFF_POW + ((CP + 2) * 4 + 15) / 16 * 16;
  static constexpr int OFF_COLF = OFF_ROWF + 4 * CP;
  // output epilogue: gate partial dots [CP][DK/8], per-row partial sums of
  // squares [CP][NWP], the gates [CP] and the per-head channel scales [DK]
  static constexpr int NWP = (NW + 3) / 4 * 4;
  static constexpr int OFF_GP = OFF_COLF + 4 * CP;
  static constexpr int OFF_SQ = OFF_GP + (EPI ? 4 * CP * (DK / 8) : 0);
  static constexpr int OFF_GATE = OFF_SQ + (EPI ? 4 * CP * NWP : 0);
  static constexpr int OFF_AUG = OFF_GATE + (EPI ? 4 * CP : 0);
  static constexpr int OFF_XCH = (OFF_AUG + (EPI ? 4 * DK : 0) + 15) / 16 * 16;
  static constexpr int BYTES = OFF_XCH + XCH_BYTES;
  static_assert(OFF_K % 16 == 0 && OFF_V % 16 == 0 && OFF_POW % 16 == 0, "LDS regions must stay aligned");
};

// One chunk pass for workgroup slot xb of a launch (the whole body of the
// kernels below).  SO (state only): the segment state pass -- only the state
// update runs, from a zero state, and the segment's end state goes to
// a.seg_state.  MRG: the earlier segments' states are written in this same
// launch, by other workgroups on this XCD, and read from L2; wait_entry()
// returns once they are all available (where it is called: see the chunk-loop
// prologue).
// Whether a one-launch full pass requests its own loads before its wait
// (see chunk_body): where its registers allow it.
constexpr bool seg_early_loads(int NW, int NT, int DK) { return NW <= 8 && NT == 1 && DK <= 128; }

struct NoWait {
  __device__ void operator()() const {}
};

template <int DK, int DV, int BN, int NW, int C, int NT, bool REV, bool SO, bool EPI = false, bool PACKED = false,
          bool MRG = false, typename Wait = NoWait>
__device__ __forceinline__ void chunk_body(const ChunkArgs& a, const int xb, char* const smem,
                                           const Wait& wait_entry = Wait{}) {
  using Lds = ChunkLds<DK, BN, C, NT, NW, EPI>;
  constexpr int NTHR = NW * 64;
  // Row split (RS > 1): RS waves share each 16-column strip, wave half rh
  // owning state rows [rh DK / RS, (rh + 1) DK / RS) -- their readouts are
  // partial sums over those rows, combined through LDS, and the chunk's row
  // tiles (intra term, output) are divided between them.
  constexpr int RS = Lds::RS;
  constexpr int NWS = NW / RS;         // waves per row half (strip owners)
  constexpr int NS = BN / (16 * NWS);  // 16-column strips per wave
  static_assert(NS >= 1 && NS * 16 * NWS == BN && NWS * RS == NW, "BN must split into 16-wide strips per wave");
  static_assert(DV % BN == 0, "DV must be a multiple of BN");
  static_assert(DK % 16 == 0 && C % 16 == 0, "dims must be multiples of 16");
  constexpr int NBLK = DV / BN;
  constexpr int CP = Lds::CP;
  constexpr int DKP = Lds::DKP;
  constexpr int NTP = Lds::NTP;
  constexpr int NTS = NT == 3 ? 3 : 2;      // terms of state fragments
  constexpr int NTK = NT == 3 ? 3 : 2;      // terms of decay-scaled values
  constexpr int PQ = Lds::PQ;
  constexpr int PK = Lds::PK;
  constexpr int PVV = Lds::PVV;
  constexpr bool SWK = Lds::SWK;
  constexpr bool SWV = Lds::SWV;
  constexpr int PP = Lds::PP;
  constexpr int DKT = DK / 16;  // 16-row tiles of the state
  constexpr int KSD = DKP / 32;  // 32-deep k-steps over DK
  constexpr int DKTO = DKT / RS;  // state row tiles owned by one wave
  constexpr int KSDO = KSD / RS;  // readout k-steps of one wave
  static_assert(RS == 1 || (DK % (32 * RS) == 0 && DKTO * RS == DKT && KSDO * RS == KSD),
                "a row split must give each half whole 32-row k-steps");
  static_assert(RS <= 2, "row tiles are divided between two halves");
  static_assert(RS == 1 || !EPI, "the fused epilogue needs whole rows per wave");
  constexpr int CT = CP / 16;    // 16-row tiles of a chunk
  constexpr int KSC = CP / 32;   // 32-deep k-steps over the chunk
  constexpr int NPT = CT * (CT + 1) / 2;  // causal P tiles
  constexpr int MAXPT = (NPT + NW - 1) / NW;
  constexpr bool TIGHT = DK > 128;  // register-tight shape: pin the schedule
  constexpr bool ALIAS_P = Lds::ALIAS_P;
  constexpr int OP2 = Lds::OP2;
  constexpr int OP4 = Lds::OP4;
  constexpr bool STG_IN_P = Lds::STG_IN_P;
  constexpr int Q_ELEMS = Lds::Q_ELEMS;
  bf16_t* const sQP = reinterpret_cast<bf16_t*>(smem);
  bf16_t* const sK = reinterpret_cast<bf16_t*>(smem + Lds::OFF_K);
  bf16_t* const sV = reinterpret_cast<bf16_t*>(smem + Lds::OFF_V);
  float* const sPow = reinterpret_cast<float*>(smem + Lds::OFF_POW);
  // per-chunk factor tables for a chunk of L tokens: row factors (how the
  // entry state reaches row i) and column factors (how row j's key/value pair
  // reaches the exit state); zero beyond L
  float* const sRowF = reinterpret_cast<float*>(smem + Lds::OFF_ROWF);
  float* const sColF = reinterpret_cast<float*>(smem + Lds::OFF_COLF);
  // output epilogue (EPI): the workgroup owns every column of its head
  static_assert(!EPI || (NBLK == 1 && !REV && !Lds::ALIAS_P), "the epilogue needs whole heads, forward time");
  constexpr int NWP = Lds::NWP;
  constexpr int PPR = DK / 8;  // 8-element parts of a row in the gate dot
  float* const sGP = reinterpret_cast<float*>(smem + Lds::OFF_GP);
  float* const sSq = reinterpret_cast<float*>(smem + Lds::OFF_SQ);
  float* const sGate = reinterpret_cast<float*>(smem + Lds::OFF_GATE);
  float* const sAug = reinterpret_cast<float*>(smem + Lds::OFF_AUG);
  bf16_t* const sQ = sQP;
  bf16_t* const sP = ALIAS_P ? sQP : sQP + Q_ELEMS;


  // XCD-aware block decode: consecutive dispatch slots on one XCD (block ids
  // congruent mod 8) walk the segments, then the column blocks, of the same
  // (b, h), so the tiles and segment states they share are served from that
  // XCD's L2.
  const int64_t BH = a.B * a.H;
  const int xcd = xb & 7;
  const int nseg = a.nseg;
  const int slot = xb >> 3;
  const int seg = slot % nseg;
  const int slot2 = slot / nseg;
  const int64_t bh = (int64_t)(slot2 / NBLK) * 8 + xcd;
  const int nblk = slot2 % NBLK;
  if (bh >= BH) return;
  // the state pass produces what later segments (in walk order) consume
  if (SO && (REV ? seg == 0 : seg == nseg - 1)) return;
  int64_t b = bh / a.H;
  const int64_t h = bh - b * a.H;
  int64_t bhu = bh;  // the (sequence, head) unit this workgroup serves
  // Packed sequences of mixed lengths are served longest first: unit index b
  // takes the sequence of rank b in descending length order (ties by index),
  // so the long sequences start in the first dispatch wave and the short
  // ones fill in behind them.  Each workgroup ranks the lengths itself (they
  // are on the device only), N^2 / threads comparisons from an LDS copy; up
  // to 512 sequences.  Every unit is still served exactly once.  (A separate
  // instantiation, so the dense kernels' code is untouched.)
  if constexpr (PACKED) {
    if (a.B <= 512) {
    int* const s_pick = reinterpret_cast<int*>(smem);  // query-tile bytes, free until its first store
    int* const s_len = s_pick + 1;
    const int nb = (int)a.B;
    for (int j = threadIdx.x; j < nb; j += NTHR) {
      int64_t c0 = a.cu[j], c1 = a.cu[j + 1];
      c0 = c0 < 0 ? 0 : (c0 > a.T ? a.T : c0);
      c1 = c1 < c0 ? c0 : (c1 > a.T ? a.T : c1);
      s_len[j] = (int)(c1 - c0);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nb; j += NTHR) {
      const int lj = s_len[j];
      int rank = 0;
      for (int i = 0; i < nb; ++i) {
        const int li2 = s_len[i];
        rank += (li2 > lj || (li2 == lj && i < j)) ? 1 : 0;
      }
      if (rank == (int)b) s_pick[0] = j;
    }
    __syncthreads();
    b = s_pick[0];
    bhu = b * a.H + h;
    __syncthreads();  // every thread has read the pick before the tile stores reuse these bytes
    }
  }

  // this unit's tokens and state: the dense (b, h) layout, or a packed
  // sequence with its state in a pool page
  int64_t T = a.T, tbase = 0;
  const float* s_init = a.s_init ? a.s_init + bhu * (int64_t)DK * DV : nullptr;
  float* s_final = a.s_final ? a.s_final + bhu * (int64_t)DK * DV : nullptr;
  if (a.cu) {
    int64_t c0 = a.cu[b], c1 = a.cu[b + 1];
    c0 = c0 < 0 ? 0 : (c0 > a.T ? a.T : c0);
    c1 = c1 < c0 ? c0 : (c1 > a.T ? a.T : c1);
    tbase = c0;
    T = c1 - c0;
  }
  if (a.pool) {
    const int64_t ps = a.slots ? a.slots[b] : b;
    if (ps < 0 || ps >= a.num_slots) return;
    float* page = a.pool + ps * a.pool_stride_n + h * (int64_t)DK * DV;
    s_init = (a.has_state == nullptr || a.has_state[b] != 0) ? page : nullptr;
    s_final = page;
  }

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int rh = RS > 1 ? w / NWS : 0;                      // row half (row-split passes)
  const int ws = RS > 1 ? w - rh * NWS : w;                 // strip-owner index
  // Row-split passes divide the chunk's row tiles between the two halves,
  // alternating in pairs (0 and 3 to one half, 1 and 2 to the other, ...),
  // which balances the causal intra work: row tile I meets I / 2 + 1 k-steps.
  auto own_row = [&](int I) { return RS == 1 || (((I + (I >> 1)) & 1) == rh); };
  const int l = tid & 63;
  const int g = l >> 4;
  const int li = l & 15;
  constexpr bool rev = REV;  // time direction (a.reverse selected this instantiation)

  const float lam = a.lam[h];
  // (a one-launch full pass after its own state pass finds the table in LDS;
  // state passes formed during its wait write the same values)
  if (!(MRG && seg != (REV ? 0 : nseg - 1)))
    for (int n = tid; n <= CP + 1; n += NTHR) sPow[n] = lam_pow_f32(lam, n);
  // epilogue: the head's channel scales, zeroed row-sum padding, and this
  // lane's RMSNorm weights (output columns (w NS + s) 16 + 4 g + r)
  float gam[NS][4];
  if constexpr (EPI && !SO) {
    for (int n = tid; n < DK; n += NTHR) sAug[n] = a.aug[h * DK + n];
    for (int n = tid; n < CP * NWP; n += NTHR) sSq[n] = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) gam[s][r] = a.gamma[h * DV + (ws * NS + s) * 16 + 4 * g + r];
  }
  // (reads sPow: every call site is preceded by a barrier after sPow is filled)
  auto fill_factors = [&](int Lc) {
    for (int n = tid; n < CP; n += NTHR) {
      const bool in = n < Lc;
      const int er = rev ? Lc - 1 - n : n + 1;  // row exponent
      const int ec = rev ? n + 1 : Lc - 1 - n;  // column exponent
      sRowF[n] = in ? sPow[er] : 0.0f;
      sColF[n] = in ? sPow[ec] : 0.0f;
    }
  };
  // decay mask of the diagonal P tiles, per lane: forward keeps j <= i with
  // lam^(i-j), reverse keeps j >= i with lam^(j-i); i = 16 I + li, j = 16 I + 4 g + r
  // (read from the table once it is complete)
  float dmask[4] = {0.f, 0.f, 0.f, 0.f};
  // Off-diagonal P-tile factors: the exponent of tile distance d = Ip - Jp
  // >= 1 is 16 d + e with e = li - 4 g - r (reverse: 4 g + r - li), formed
  // as lam^(16 (d - 1)) times lp[r] = lam^(16 + e).  Where a wave has at
  // most two tile slots (slot kt holds the same tile in every chunk) their
  // whole factors are kept in mf instead, filled once the table is complete.
  constexpr bool MFT = !TIGHT && MAXPT <= 2 && NT == 1;
  float lp[4] = {0.f, 0.f, 0.f, 0.f};
  float mf[MFT ? MAXPT : 1][4] = {};

  const char* qb = reinterpret_cast<const char*>(a.q);
  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const int esz = a.in_f32 ? 4 : 2;
  const int64_t q_off = b * a.sq_b + h * a.sq_h + tbase * a.sq_t;
  const int64_t k_off = b * a.sk_b + h * a.sk_h + tbase * a.sk_t;
  const int64_t v_off = b * a.sv_b + h * a.sv_h + tbase * a.sv_t + (int64_t)nblk * BN;
  const int col0 = nblk * BN + ws * NS * 16 + li;  // + 16 s: this lane's column in strip s

  // A segment's end state in the workspace, in the register order of the
  // workgroups that write and read it (both run this tiling): per column
  // block, 16-byte groups (a lane's four r values) indexed by (Do, s, thread).
  auto seg_block = [&](int p) -> float* {
    return a.seg_state + ((bh * nseg + p) * NBLK + nblk) * (int64_t)(DK * BN);
  };

  // ---- state slice in accumulators: accS[Do][s][r] = S[state_row(D)][col0 + 16 s]
  // for this wave's row tiles D = rh DKTO + Do
  f32x4 accS[DKTO][NS];
  auto load_entry = [&]() {
    const float* si = SO ? nullptr : s_init;
#pragma unroll
    for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int D = rh * DKTO + Do;
          const int d = state_row<DK>(D, g, r);
          const int n = col0 + 16 * s;
          float x = 0.0f;
          if (si) x = a.s_init_trans ? si[(int64_t)n * DK + d] : si[(int64_t)d * DV + n];
          accS[Do][s][r] = x;
        }
  };
  // Workgroups of up to two waves per SIMD (bf16 tiles, DK <= 128) wait
  // inside the chunk-loop prologue (below); otherwise the tiles' registers
  // held through the wait would spill.  The last segment in walk order has
  // no state pass of its own: it requests its entry state and first tiles
  // before it waits, while the others run their state passes.  The others
  // reach the wait just as the flags are due and poll with no loads of their
  // own in flight (a wait for a load is a wait for every load issued before
  // it).
  constexpr bool EARLY = MRG && seg_early_loads(NW, NT, DK);
  const bool idle_wait = seg == (REV ? 0 : nseg - 1);
  if (!EARLY || idle_wait) load_entry();
  // The segments before this one (in walk order) enter through their end
  // states: S <- lam^len S + E, oldest first.  Every such segment is whole
  // except, in reverse time, the last one (walked first), so two powers
  // serve them all.
  auto fold_entry = [&]() {
    const int first = REV ? nseg - 1 : 0;
    const int step = REV ? -1 : 1;
    const int64_t tail = T - (int64_t)(nseg - 1) * a.seg_len;  // the last segment's length
    const float dec_full = first != seg ? lam_pow_f32(lam, (int)a.seg_len) : 1.0f;
    const float dec_last = (REV && first != seg) ? lam_pow_f32(lam, (int)tail) : dec_full;
    if constexpr (MRG) {
      // States written in this launch by other workgroups: read at device
      // scope (past this CU's cache), FB of them requested at once, then
      // folded in walk order (walk position j is segment p).
      constexpr int FB = TIGHT ? 1 : 4;
      const int nprev = REV ? nseg - 1 - seg : seg;
      for (int j0 = 0; j0 < nprev; j0 += FB) {
        f32x4 e[FB][DKTO][NS];
#pragma unroll
        for (int u = 0; u < FB; ++u) {
          if (j0 + u >= nprev) continue;
          const int p = REV ? nseg - 1 - (j0 + u) : j0 + u;
          const __amdgpu_buffer_rsrc_t rs =
              __builtin_amdgcn_make_buffer_rsrc(seg_block(p), (short)0, DK * BN * 4, 0x00020000);
#pragma unroll
          for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
            for (int s = 0; s < NS; ++s)
              e[u][Do][s] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ((Do * NS + s) * NTHR + tid) * 16, 0, kCpolSc1));
        }
#pragma unroll
        for (int u = 0; u < FB; ++u) {
          if (j0 + u >= nprev) continue;
          const float dec = (REV && j0 + u == 0) ? dec_last : dec_full;
#pragma unroll
          for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int r = 0; r < 4; ++r) accS[Do][s][r] = fmaf(dec, accS[Do][s][r], e[u][Do][s][r]);
        }
      }
    } else {
      for (int p = first; p != seg; p += step) {
        const float dec = p == nseg - 1 ? dec_last : dec_full;
        const f32x4* const E = reinterpret_cast<const f32x4*>(seg_block(p));
#pragma unroll
        for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const f32x4 x = E[(Do * NS + s) * NTHR + tid];
#pragma unroll
            for (int r = 0; r < 4; ++r) accS[Do][s][r] = fmaf(dec, accS[Do][s][r], x[r]);
          }
      }
    }
  };
  if constexpr (!SO && !MRG) fold_entry();
  if constexpr (MRG && !EARLY) {
    wait_entry();
    fold_entry();
  }

  // The entry state has landed before the chunk loop starts.  (Without this
  // explicit wait the compiler cannot prove it on every path into the loop
  // and waits for all outstanding global loads -- including the next chunk's
  // prefetch -- at the first use of the state in every iteration.)
  if constexpr (!EARLY) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt unchanged

  // writes 4 consecutive masked-P values of row i (cols 16 J + 4 g ..) as NTP planes
  auto put_p = [&](int i, int J, const f32x4& val) {
    const float x[4] = {val[0], val[1], val[2], val[3]};
    bf16x4 pk[NTP];
    split_vec<NTP>(x, pk);
#pragma unroll
    for (int p = 0; p < NTP; ++p) *reinterpret_cast<bf16x4*>(&sP[p * CP * PP + i * PP + 16 * J + 4 * g]) = pk[p];
  };
  // zero tiles read by the 32-deep k-steps of stage 3: forward (I, I+1) for
  // even I, reverse (I, I-1) for odd I
  auto put_zero_tiles = [&]() {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int zi = w; zi < CT / 2; zi += NW) {
      const int I = rev ? 2 * zi + 1 : 2 * zi;
      put_p(16 * I + li, rev ? I - 1 : I + 1, z);
    }
  };

  // this segment's tokens [tb, te) and their chunks
  const int64_t tb = (int64_t)seg * a.seg_len;
  const int64_t te = (T - tb) < a.seg_len ? T : tb + a.seg_len;
  const int64_t nchunks = (te - tb + C - 1) / C;
  // chunk ci of the walk (reverse time walks the chunks backwards)
  auto chunk_start = [&](int64_t ci) { return tb + (rev ? (nchunks - 1 - ci) : ci) * C; };
  auto chunk_len = [&](int64_t t0) { return (int)((te - t0) < C ? (te - t0) : C); };

  // The next chunk's tiles are loaded into registers while the current chunk
  // is computed, so HBM latency overlaps the MFMA work.
  TileStager<NT, CP, DK, DKP, PQ, NTHR> pfq;
  TileStager<NT, CP, DK, DKP, PK, NTHR, SWK> pfk;
  TileStager<NT, CP, BN, BN, PVV, NTHR, SWV> pfv;
  // With wide query/key rows (192 channels) the next query tile is fetched
  // only after stage 2: holding it through the P tiles and the readout keeps
  // 16 more registers live at the register peak, and the earlier fetch
  // measured slower.
  constexpr bool LATE_Q = DK > 128;
  auto prefetch_q = [&](int64_t ci) {
    const int64_t t0 = chunk_start(ci);
    pfq.load(qb + (q_off + t0 * a.sq_t) * esz, (uint32_t)a.sq_t, chunk_len(t0), tid);
  };
  auto prefetch_kv = [&](int64_t ci) {
    const int64_t t0 = chunk_start(ci);
    const int Ln = chunk_len(t0);
    pfk.load(kb + (k_off + t0 * a.sk_t) * esz, (uint32_t)a.sk_t, Ln, tid);
    pfv.load(vb + (v_off + t0 * a.sv_t) * esz, (uint32_t)a.sv_t, Ln, tid);
  };
  // Stores a staged output chunk (tokens [t0s, t0s + Ls) of this unit's
  // column block) with coalesced 16-byte row writes.  accO held O^T tiles:
  // lane (g, li) had row 16 I + li, columns strip + 4 g .. + 3, and the
  // staging buffer holds them row-major.  The buffer resource ends at the
  // last valid row, so stores of rows >= Ls are dropped by the hardware
  // range check.
  auto store_out = [&](const bf16_t* stg, int64_t t0s, int Ls) {
    const int f32o = a.o_f32;
    const int oes = f32o ? 4 : 2;
    char* obase = reinterpret_cast<char*>(a.o) + (b * a.so_b + h * a.so_h + (tbase + t0s) * a.so_t + nblk * BN) * oes;
    const uint32_t so_t = (uint32_t)a.so_t;
    const uint32_t nbytes = ((uint32_t)(Ls - 1) * so_t + BN) * oes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(obase, (short)0, (int)nbytes, 0x00020000);
    // thread tid stores column vector tid % VPR of rows tid / VPR + RPJ j
    auto store_rows = [&](auto vpr_c, auto es_c) {
      constexpr int VPR = decltype(vpr_c)::value;  // 16-byte vectors per row
      constexpr int ES = decltype(es_c)::value;
      static_assert(NTHR % VPR == 0, "threads must cover whole rows");
      constexpr int RPJ = NTHR / VPR;
      constexpr int PITCH_B = ES == 4 ? OP4 * 4 : OP2 * 2;  // staging pitch in bytes
      const int row0 = tid / VPR;
      const int cv = tid - row0 * VPR;
      const char* src = reinterpret_cast<const char*>(stg) + row0 * PITCH_B + cv * 16;
      const uint32_t voff = (uint32_t)row0 * so_t * ES + cv * 16;
#pragma unroll
      for (int j = 0; j < (CP + RPJ - 1) / RPJ; ++j) {
        if (CP % RPJ == 0 || row0 + j * RPJ < CP) {
          const u32x4 val = *reinterpret_cast<const u32x4*>(src + j * RPJ * PITCH_B);
          __builtin_amdgcn_raw_buffer_store_b128(val, rs, voff, (int)((uint32_t)(j * RPJ) * so_t * ES), 0);
        }
      }
    };
    if (f32o) store_rows(std::integral_constant<int, BN * 4 / 16>{}, std::integral_constant<int, 4>{});
    else store_rows(std::integral_constant<int, BN * 2 / 16>{}, std::integral_constant<int, 2>{});
  };

  // Chunk pipeline.  The tiles of chunk ci+1 are loaded into registers while
  // chunk ci is computed and written to LDS as soon as its last reader is
  // done; the output of chunk ci is stored last, so its write latency
  // overlaps the compute of chunk ci+1.
  if constexpr (EARLY) {
    if (nchunks > 0 && idle_wait) {
      prefetch_q(0);
      prefetch_kv(0);
    }
    wait_entry();
    if (!idle_wait) {
      load_entry();
      if (nchunks > 0) {
        prefetch_q(0);
        prefetch_kv(0);
      }
    }
    fold_entry();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): entry state and first tiles
  }
  if (nchunks > 0) {
    if constexpr (!EARLY) {
      if constexpr (!SO) prefetch_q(0);
      prefetch_kv(0);
    }
    if constexpr (!SO) pfq.store(sQ, tid);
    pfk.store(sK, tid);
    pfv.store(sV, tid);
    __syncthreads();  // sPow complete
    fill_factors(chunk_len(chunk_start(0)));
    if constexpr (!SO) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = rev ? (4 * g + r - li) : (li - 4 * g - r);
        dmask[r] = d >= 0 ? sPow[d] : 0.0f;
      }
    }
    if constexpr (!TIGHT) {
#pragma unroll
      for (int r = 0; r < 4; ++r) lp[r] = sPow[16 + (rev ? 4 * g + r - li : li - 4 * g - r)];
    }
    if constexpr (MFT) {
#pragma unroll
      for (int kt = 0; kt < MAXPT; ++kt) {
        const int t = w + kt * NW;
        int Ip, Jp;
        tile_of<CT>(t < NPT ? t : 0, Ip, Jp);
        const int d = Ip - Jp;
        const float s16 = sPow[16 * (d > 0 ? d - 1 : 0)];
#pragma unroll
        for (int r = 0; r < 4; ++r) mf[kt][r] = d == 0 ? dmask[r] : s16 * lp[r];
      }
    }
  }

  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = chunk_start(ci);
    const int L = chunk_len(t0);

    // ---------------- stage 0: this chunk's tiles are in LDS; start the next loads
    __syncthreads();
    if (ci + 1 < nchunks) {
      if constexpr (!LATE_Q && !SO) prefetch_q(ci + 1);
      prefetch_kv(ci + 1);
    }

    // ---------------- stage 1: masked P tiles (causal half), P[i][j] row-major
    // Each wave computes the tiles t = w, w + NW, ..., TP of them at a time so
    // their LDS reads and MFMA chains overlap.  Slots past the last tile are
    // skipped (the wave index is uniform, so this is a scalar branch): when the
    // tiles do not divide evenly the waves that run out are those after the
    // first NPT % NW, i.e. the second waves on SIMDs 0 and 1, which carry the
    // longest path through the chunk.
    f32x4 ptile[ALIAS_P ? MAXPT : 1];
    if constexpr (!SO) {
      constexpr int TP = (TIGHT || MAXPT < 2) ? 1 : 2;
      auto p_batch = [&](auto tp_c, const int kt0) {
        constexpr int TB = decltype(tp_c)::value;  // tiles in this batch, all valid
        int Ia[TB], Ja[TB], da[TB];
        f32x4 acc[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const int t = w + (kt0 + u) * NW;
          int Ip, Jp;
          tile_of<CT>(t, Ip, Jp);
          Ia[u] = rev ? CT - 1 - Ip : Ip;
          Ja[u] = rev ? CT - 1 - Jp : Jp;
          da[u] = Ip - Jp;
          acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          bf16x8 A[TB][NT], Bq[TB][NT];
#pragma unroll
          for (int u = 0; u < TB; ++u)
#pragma unroll
            for (int p = 0; p < NT; ++p) {
              A[u][p] = lds_read_b128(&sK[p * CP * PK + (16 * Ja[u] + li) * PK + 32 * ks +
                                          (SWK ? 8 * g ^ tile_swz(li) : 8 * g)]);
              Bq[u][p] = lds_read_b128(&sQ[p * CP * PQ + (16 * Ia[u] + li) * PQ + 32 * ks + 8 * g]);
            }
#pragma unroll
          for (int u = 0; u < TB; ++u) mma_split<NT, NT>(acc[u], A[u], Bq[u]);
        }
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          // acc[r] = q'_i . k'_j with i = 16 I + li, j = 16 J + 4 g + r, times
          // its decay mask (register-tight shapes read the whole exponent
          // 16 d + base -/+ r from the table)
          if constexpr (TIGHT) {
            const int base = 16 * da[u] + (rev ? 4 * g - li : li - 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[u][r] *= da[u] == 0 ? dmask[r] : sPow[da[u] == 0 ? 0 : (rev ? base + r : base - r)];
          } else if constexpr (MFT) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] *= mf[kt0 + u][r];
          } else {
            const float s16 = sPow[16 * (da[u] > 0 ? da[u] - 1 : 0)];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] *= da[u] == 0 ? dmask[r] : s16 * lp[r];
          }
          if constexpr (ALIAS_P) ptile[kt0 + u] = acc[u];
          else put_p(16 * Ia[u] + li, Ja[u], acc[u]);
        }
        if constexpr (TIGHT) __builtin_amdgcn_sched_barrier(0);
      };
      // slot kt is valid iff w + kt NW < NPT; valid slots come first
      auto slot_ok = [&](int kt) { return kt < MAXPT && (NPT % NW == 0 || w + kt * NW < NPT); };
#pragma unroll
      for (int kt0 = 0; kt0 < MAXPT; kt0 += TP) {
        if constexpr (NPT % NW == 0 && MAXPT % TP == 0) {
          p_batch(std::integral_constant<int, TP>{}, kt0);  // every slot is a tile
        } else if constexpr (TP == 2) {
          if (slot_ok(kt0 + 1)) p_batch(std::integral_constant<int, 2>{}, kt0);
          else if (slot_ok(kt0)) p_batch(std::integral_constant<int, 1>{}, kt0);
        } else {
          if (slot_ok(kt0)) p_batch(std::integral_constant<int, 1>{}, kt0);
        }
      }
      if constexpr (!ALIAS_P) put_zero_tiles();
    }

    // ---------------- stage 2: O^T = S^T Q^T, rows scaled by the row factors
    f32x4 accO[CT][NS];
#pragma unroll
    for (int I = 0; I < CT; ++I)
#pragma unroll
      for (int s = 0; s < NS; ++s) accO[I][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!SO) {
#pragma unroll
    for (int kso = 0; kso < KSDO; ++kso) {
      // State as the B operand of Q S: k-slot e of lane group g takes
      // accumulator slot e % 4 of row tile 2 ks + e / 4, i.e. state row
      // state_row(2 ks + e / 4, g, e % 4); Q is read at the same rows
      // (32 ks + 8 g + e when DK is a multiple of 32).  A row-split wave
      // covers only its own k-steps.
      const int ks = rh * KSDO + kso;
      bf16x8 Sf[NS][NTS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int Do = 2 * kso + (e >> 2);
          x[e] = (Do < DKTO) ? accS[Do < DKTO ? Do : 0][s][e & 3] : 0.0f;
        }
        split_vec<NTS>(x, Sf[s]);
      }
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        bf16x8 Aq[NT];
        const int Iph = rev ? CT - 1 - I : I;  // accO[I] holds physical row tile Iph
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          const bf16_t* row = &sQ[p * CP * PQ + (16 * Iph + li) * PQ + 32 * ks];
          if constexpr (DK % 32 == 0) Aq[p] = lds_read_b128(row + 8 * g);
          else Aq[p] = cat4(lds_read_b64(row + 4 * g), lds_read_b64(row + 16 + 4 * g));
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) mma_split<NTS, NT>(accO[I][s], Sf[s], Aq);
        if constexpr (TIGHT) {
          if (I % 4 == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    }
    {
      const float cfac = sPow[L];
#pragma unroll
      for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) accS[Do][s][r] *= cfac;
      if constexpr (!SO) {
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          const int i = 16 * (rev ? CT - 1 - I : I) + li;
          const float f = sRowF[i];
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) accO[I][s][r] *= f;
        }
      }
    }

    // row split: hand the partial readout of the other half's row tiles over
    float* const sX = reinterpret_cast<float*>(smem + Lds::OFF_XCH);
    if constexpr (RS > 1 && !SO) {
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        if (own_row(I)) continue;
        const int row = 16 * (rev ? CT - 1 - I : I) + li;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          *reinterpret_cast<f32x4*>(&sX[row * Lds::XP + (ws * NS + s) * 16 + 4 * g]) = accO[I][s];
      }
    }
    if constexpr (ALIAS_P && !SO) {
      __syncthreads();  // every read of the query tile is done
#pragma unroll
      for (int kt = 0; kt < MAXPT; ++kt) {
        const int t = w + kt * NW;
        if (NPT % NW == 0 || t < NPT) {
          int Ip, Jp;
          tile_of<CT>(t, Ip, Jp);
          const int I = rev ? CT - 1 - Ip : Ip;
          const int J = rev ? CT - 1 - Jp : Jp;
          put_p(16 * I + li, J, ptile[kt]);
        }
      }
      put_zero_tiles();
    }
    if constexpr (EPI && !SO) {
      // self-augmentation gate: partial dots q_i . (aug * k_i) over 8 channels
      for (int u = tid; u < CP * PPR; u += NTHR) {
        const int row = u / PPR;
        const int part = u - row * PPR;
        bf16x8 qp[NT], kp[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          qp[p] = lds_read_b128(&sQ[p * CP * PQ + row * PQ + part * 8]);
          kp[p] = lds_read_b128(&sK[p * CP * PK + row * PK + (SWK ? part * 8 ^ tile_swz(row) : part * 8)]);
        }
        float sacc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float qe = 0.0f, ke = 0.0f;
#pragma unroll
          for (int p = 0; p < NT; ++p) {
            qe += bf16v_to_f32(qp[p][e]);
            ke += bf16v_to_f32(kp[p][e]);
          }
          sacc = fmaf(qe * sAug[part * 8 + e], ke, sacc);
        }
        sGP[u] = sacc;
      }
    }
    if constexpr (!SO) __syncthreads();  // P complete (and the readout hand-over)
    // wide query rows: the next query tile is fetched now, once the readout's
    // registers are free, and written to LDS at the end of the chunk
    if constexpr (LATE_Q && !SO) {
      if (ci + 1 < nchunks) prefetch_q(ci + 1);
    }
    // row split: add the other half's partial readout of this wave's row tiles
    if constexpr (RS > 1 && !SO) {
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        if (!own_row(I)) continue;
        const int row = 16 * (rev ? CT - 1 - I : I) + li;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(&sX[row * Lds::XP + (ws * NS + s) * 16 + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) accO[I][s][r] += t[r];
        }
      }
    }
    if constexpr (EPI && !SO) {
      for (int row = tid; row < CP; row += NTHR) {
        float sdot = 0.0f;
        for (int part = 0; part < PPR; ++part) sdot += sGP[row * PPR + part];
        sGate[row] = sigmoid_hw(sdot);
      }
    }

    // ---------------- stage 3: O += P V ; stage 4: S += (colfac K)^T V
    // Logical k-steps kl and row tiles I keep the causal structure static:
    // physical k-step ks = rev ? KSC-1-kl : kl, physical row tile
    // rev ? CT-1-I : I, and row tile I meets k-step kl iff kl <= I / 2.
    auto kstep = [&](const int kl) {
      const int ks = rev ? KSC - 1 - kl : kl;
      // V fragments: B[k = 32 ks + 8 g + e][n = strip col + li] via column reads
      bf16x8 Bv[NS][NT];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        // rows 32 ks + 8 g + (0..7): bit 3 is that of 8 g
        const int c0 = ((ws * NS + s) * 16 + 4 * (li & 3)) ^ (SWV ? tile_swz(8 * g) : 0);
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          const bf16_t* base = &sV[p * CP * PVV + (32 * ks + 8 * g + (li >> 2)) * PVV + c0];
          Bv[s][p] = cat4(lds_read_tr(base), lds_read_tr(base + 4 * PVV));
        }
      }
      // stage 3 for the row tiles whose causal window touches this k-step
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        if (SO || kl > (I >> 1) || !own_row(I)) continue;
        const int Iph = rev ? CT - 1 - I : I;
        bf16x8 Ap[NTP];
#pragma unroll
        for (int p = 0; p < NTP; ++p)
          Ap[p] = lds_read_b128(&sP[p * CP * PP + (16 * Iph + li) * PP + 32 * ks + 8 * g]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma_split<NT, NTP>(accO[I][s], Bv[s], Ap);
        if constexpr (TIGHT) __builtin_amdgcn_sched_barrier(0);
      }
      // stage 4: S += K^T (diag(col factors) V).  The decay rides on this
      // wave's own value strip (split hi/lo); the keys enter exact.
      bf16x8 Bs[NS][NTK];
      {
        const f32x4 cf0 = *reinterpret_cast<const f32x4*>(&sColF[32 * ks + 8 * g]);
        const f32x4 cf1 = *reinterpret_cast<const f32x4*>(&sColF[32 * ks + 8 * g + 4]);
        const float cf[8] = {cf0[0], cf0[1], cf0[2], cf0[3], cf1[0], cf1[1], cf1[2], cf1[3]};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float v = bf16v_to_f32(Bv[s][0][e]);
#pragma unroll
            for (int p = 1; p < NT; ++p) v += bf16v_to_f32(Bv[s][p][e]);
            x[e] = v * cf[e];
          }
          split_vec<NTK>(x, Bs[s]);
        }
      }
#pragma unroll
      for (int Do = 0; Do < DKTO; ++Do) {
        const int D = rh * DKTO + Do;  // this wave's state row tiles
        // keys as the A operand, A[m = d][k = j], via column reads
        bf16x8 Ak[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          // lane li supplies the 4-column group that lanes 4 (li & 3) .. + 3
          // receive: their state rows (state_row) select the key columns
          const int kc = (DK % 32 == 0 ? 32 * (D >> 1) + 8 * (li & 3) + 4 * (D & 1) : 16 * D + 4 * (li & 3)) ^
                         (SWK ? tile_swz(8 * g) : 0);
          const bf16_t* base = &sK[p * CP * PK + (32 * ks + 8 * g + (li >> 2)) * PK + kc];
          Ak[p] = cat4(lds_read_tr(base), lds_read_tr(base + 4 * PK));
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) mma_split<NT, NTK>(accS[Do][s], Ak, Bs[s]);
        // where registers are tight, keep the scheduler from hoisting every
        // tile's loads at once
        if constexpr (TIGHT) __builtin_amdgcn_sched_barrier(0);
      }
      // one k-step at a time: bounds the loads in flight, hence the registers
      __builtin_amdgcn_sched_barrier(0);
        };
    // where registers are tight, walk the k-steps as a loop; else unroll them
    if constexpr (TIGHT) {
#pragma unroll 1
      for (int kl = 0; kl < KSC; ++kl) kstep(kl);
    } else {
#pragma unroll
      for (int kl = 0; kl < KSC; ++kl) kstep(kl);
    }

    // epilogue: this lane's values v[16 I + li][(w NS + s) 16 + 4 g + r],
    // read while the value tile is still in LDS
    float vreg[EPI ? CT : 1][NS][4];
    if constexpr (EPI && !SO) {
#pragma unroll
      for (int I = 0; I < CT; ++I)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
          for (int r = 0; r < 4; ++r) vreg[I][s][r] = 0.0f;
#pragma unroll
          for (int p = 0; p < NT; ++p) {
            const bf16x4 t = lds_read_b64(&sV[p * CP * PVV + (16 * I + li) * PVV +
                                              (((ws * NS + s) * 16 + 4 * g) ^ (SWV ? tile_swz(li) : 0))]);
#pragma unroll
            for (int r = 0; r < 4; ++r) vreg[I][s][r] += bf16v_to_f32(t[r]);
          }
        }
    }

    // ---------------- next chunk's tiles -> LDS; store O (rows < L)
    // O is staged through LDS so that the global stores are 16-byte,
    // row-contiguous and coalesced.  accO holds O^T tiles: lane (g, li) has
    // row 16 I + li, columns strip + 4 g .. + 3.  The staging buffer is the P
    // region when it fits, else the query+P region (then the next chunk's
    // tiles are written only after the staged output has been read).  The
    // buffer resource ends at the last valid row, so stores of rows >= L are
    // dropped by the hardware range check.
    __syncthreads();  // every wave is done with the P, key and value tiles
    const bool more = ci + 1 < nchunks;
    // the factor tables change only when the next chunk's length differs
    const bool refill = more && chunk_len(chunk_start(ci + 1)) != L;
    // this wave's output rows into the staging buffer: fp32, or bf16 rounded
    // to nearest
    auto stage_out = [&](bf16_t* stg) {
      if (a.o_f32) {
        float* st4 = reinterpret_cast<float*>(stg);
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          if (!own_row(I)) continue;
#pragma unroll
          for (int s = 0; s < NS; ++s)
            *reinterpret_cast<f32x4*>(&st4[(16 * (rev ? CT - 1 - I : I) + li) * OP4 + (ws * NS + s) * 16 + 4 * g]) =
                accO[I][s];
        }
      } else {
#pragma unroll
        for (int I = 0; I < CT; ++I) {
          if (!own_row(I)) continue;
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            bf16x4 pk;
#pragma unroll
            for (int r = 0; r < 4; ++r) pk[r] = (__bf16)accO[I][s][r];
            *reinterpret_cast<bf16x4*>(&stg[(16 * (rev ? CT - 1 - I : I) + li) * OP2 + (ws * NS + s) * 16 + 4 * g]) = pk;
          }
        }
      }
    };
    if (more) {
      pfk.store(sK, tid);
      pfv.store(sV, tid);
      if constexpr (STG_IN_P && !LATE_Q && !SO) pfq.store(sQ, tid);
    }
    if constexpr (STG_IN_P) {
      if (refill) fill_factors(chunk_len(chunk_start(ci + 1)));
    }
    if constexpr (EPI && !SO) {
      // this chunk's gate-stream values for the store below, loaded now so
      // their latency overlaps the normalisation (8 columns per thread)
      const int ges = a.in_f32 ? 4 : 2;
      const char* gbase =
          reinterpret_cast<const char*>(a.gz) + (b * a.sg_b + h * a.sg_h + (tbase + t0) * a.sg_t) * ges;
      const __amdgpu_buffer_rsrc_t rsg = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(gbase), (short)0, (int)(((uint32_t)(L - 1) * (uint32_t)a.sg_t + BN) * ges), 0x00020000);
      constexpr int VPR8 = BN / 8;
      static_assert(NTHR % VPR8 == 0, "threads must cover whole rows");
      constexpr int RPJ8 = NTHR / VPR8;
      constexpr int NJ8 = (CP + RPJ8 - 1) / RPJ8;
      const int row0 = tid / VPR8;
      const int cv = tid - row0 * VPR8;
      u32x4 graw[NJ8][NT == 3 ? 2 : 1];
#pragma unroll
      for (int j = 0; j < NJ8; ++j) {
        const int row = row0 + j * RPJ8;
        if (CP % RPJ8 == 0 || row < CP) {
          if constexpr (NT == 3) {
            const uint32_t go = (uint32_t)row * (uint32_t)a.sg_t * 4 + cv * 32;
            graw[j][0] = __builtin_amdgcn_raw_buffer_load_b128(rsg, go, 0, 0);
            graw[j][1] = __builtin_amdgcn_raw_buffer_load_b128(rsg, go + 16, 0, 0);
          } else {
            graw[j][0] = __builtin_amdgcn_raw_buffer_load_b128(rsg, (uint32_t)row * (uint32_t)a.sg_t * 2 + cv * 16, 0, 0);
          }
        }
      }
      // o' = o + gate v, then per-row sums of squares over this wave's columns
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        const int row = 16 * I + li;
        const float gt = sGate[row];
        float ss = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            accO[I][s][r] = fmaf(gt, vreg[I][s][r], accO[I][s][r]);
            ss = fmaf(accO[I][s][r], accO[I][s][r], ss);
          }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (g == 0) sSq[row * NWP + w] = ss;
      }
      __syncthreads();  // row sums complete
      // Head RMSNorm and its weight; staged in fp32
      float* st4 = reinterpret_cast<float*>(STG_IN_P ? sP : sQP);
#pragma unroll
      for (int I = 0; I < CT; ++I) {
        const int row = 16 * I + li;
        float tot = 0.0f;
#pragma unroll
        for (int v4 = 0; v4 < NWP; v4 += 4) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(&sSq[row * NWP + v4]);
          tot += (t[0] + t[1]) + (t[2] + t[3]);
        }
        const float rstd = __builtin_amdgcn_rsqf(tot * (1.0f / DV) + a.eps);  // hardware 1/sqrt, ~1 ulp
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          f32x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = accO[I][s][r] * rstd * gam[s][r];
          *reinterpret_cast<f32x4*>(&st4[row * OP4 + (ws * NS + s) * 16 + 4 * g]) = y;
        }
      }
      __syncthreads();
      // y * SiLU(gate stream): 8 columns per thread, coalesced 16-byte rows
      const int oes = a.o_f32 ? 4 : 2;
      char* obase = reinterpret_cast<char*>(a.o) + (b * a.so_b + h * a.so_h + (tbase + t0) * a.so_t) * oes;
      const __amdgpu_buffer_rsrc_t rso = __builtin_amdgcn_make_buffer_rsrc(
          obase, (short)0, (int)(((uint32_t)(L - 1) * (uint32_t)a.so_t + BN) * oes), 0x00020000);
#pragma unroll
      for (int j = 0; j < NJ8; ++j) {
        const int row = row0 + j * RPJ8;
        if (CP % RPJ8 == 0 || row < CP) {
          const f32x4 y0 = *reinterpret_cast<const f32x4*>(&st4[row * OP4 + cv * 8]);
          const f32x4 y1 = *reinterpret_cast<const f32x4*>(&st4[row * OP4 + cv * 8 + 4]);
          float gv[8];
          if constexpr (NT == 3) {
            const f32x4 g0 = __builtin_bit_cast(f32x4, graw[j][0]);
            const f32x4 g1 = __builtin_bit_cast(f32x4, graw[j][NT == 3 ? 1 : 0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              gv[e] = g0[e];
              gv[4 + e] = g1[e];
            }
          } else {
            const bf16x8 gb = __builtin_bit_cast(bf16x8, graw[j][0]);
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[e] = bf16v_to_f32(gb[e]);
          }
          float out[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float yv = e < 4 ? y0[e] : y1[e - 4];
            out[e] = yv * gv[e] * sigmoid_hw(gv[e]);
          }
          if (a.o_f32) {
            const uint32_t oo = (uint32_t)row * (uint32_t)a.so_t * 4 + cv * 32;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{out[0], out[1], out[2], out[3]}), rso, oo, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{out[4], out[5], out[6], out[7]}), rso, oo + 16, 0, 0);
          } else {
            bf16x8 pk;
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[e] = (__bf16)out[e];
            const uint32_t oo = (uint32_t)row * (uint32_t)a.so_t * 2 + cv * 16;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pk), rso, oo, 0, 0);
          }
        }
      }
    } else if constexpr (!SO) {
      bf16_t* stg = STG_IN_P ? sP : sQP;
      stage_out(stg);
      __syncthreads();
      store_out(stg, t0, L);
    }
    if constexpr (!STG_IN_P) {
      __syncthreads();  // the staged output has been read
      if (refill) fill_factors(chunk_len(chunk_start(ci + 1)));
    }
    if constexpr ((!STG_IN_P || LATE_Q) && !SO) {
      if (more) pfq.store(sQ, tid);
    }
  }

  // the state pass hands its segment's end state to the later segments (in
  // register order); the last segment in walk order returns the final state
  if constexpr (SO) {
    f32x4* const E = reinterpret_cast<f32x4*>(seg_block(seg));
#pragma unroll
    for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
      for (int s = 0; s < NS; ++s) E[(Do * NS + s) * NTHR + tid] = accS[Do][s];
  } else if (s_final && seg == (REV ? 0 : nseg - 1)) {
#pragma unroll
    for (int Do = 0; Do < DKTO; ++Do)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s_final[(int64_t)state_row<DK>(rh * DKTO + Do, g, r) * DV + col0 + 16 * s] = accS[Do][s][r];
  }
}

template <int DK, int DV, int BN, int NW, int C, int NT, bool REV, bool SO, bool EPI = false, bool PACKED = false>
__global__ void __launch_bounds__(NW * 64) chunk_kernel(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[ChunkLds<DK, BN, C, NT, NW, EPI>::BYTES];
  chunk_body<DK, DV, BN, NW, C, NT, REV, SO, EPI, PACKED>(a, blockIdx.x, smem);
}

// Hardware id of the XCD (its own L2) that runs this workgroup.
__device__ __forceinline__ unsigned xcc_id() {
  return __builtin_amdgcn_s_getreg(20 /* XCC_ID */ | (0 << 6) | ((4 - 1) << 11)) & 0xfu;
}

// A segment split in one launch.  Workgroup (unit, segment) first runs its
// segment's state pass and publishes the end state (stores drained to L2,
// then the flag).  Its full pass then waits for the earlier segments (the
// last segment, which has no state pass, fills its tables and requests its
// entry state and first tiles first): lane p of wave 0 polls the flag of
// walk position p, whose workgroup sits 8 (segment distance) block
// ids away (earlier in forward time, later in reverse time) and so --
// workgroups being dealt to the XCDs in turn -- on the same XCD, sharing its
// L2.  (The launch is used only when every workgroup has a compute unit of
// its own, so all are resident.)  A flag counts only if it carries this call's
// tag and this XCD's id.  Any earlier state not published within a.seg_wait
// ticks (the producer not resident, or on another XCD) is formed here by the
// same state pass, bit for bit what its producer writes.  Then the full pass
// folds them in as in the two-launch form.  Every wait is bounded, so the
// launch completes whatever the residency; the flags are cleared on exit so a
// graph replay (same tag) starts from clear flags.
template <int DK, int DV, int BN, int NW, int C, int NT, bool REV>
__device__ __forceinline__ void seg_pass(const ChunkArgs& a, const int xb, char* const smem,
                                         unsigned long long& s_todo) {
  constexpr int NBLK = DV / BN;
  const int nseg = a.nseg;
  const int seg = (xb >> 3) % nseg;
  const int slot2 = (xb >> 3) / nseg;
  const int64_t bh = (int64_t)(slot2 / NBLK) * 8 + (xb & 7);
  if (bh >= a.B * a.H) return;
  unsigned long long* const flag = a.seg_flag + (bh * NBLK + slot2 % NBLK) * nseg;
  const int wi = REV ? nseg - 1 - seg : seg;  // position in walk order
  const unsigned long long tag = a.seg_tag | xcc_id();
  // this segment's end state from a zero start (the last segment in walk
  // order has none), published once its stores are in L2
  if (wi < nseg - 1) {
    chunk_body<DK, DV, BN, NW, C, NT, REV, true>(a, xb, smem);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's state stores are in L2
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag + seg, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // LDS free for the full pass
  }
  // Called by the full pass (or before it): returns once every earlier state
  // is published here, or formed by this workgroup.
  auto wait_entry = [&]() {
    if (threadIdx.x < 64) {  // wave 0, lane p polls the flag of walk position p
      const int p = threadIdx.x;
      const int sp = REV ? nseg - 1 - p : p;
      bool done = p >= wi, miss = false;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (int it = 0;; ++it) {
        if (!done) {
          const unsigned long long f = __hip_atomic_load(flag + sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (f == tag) {
            done = true;
          } else if ((f & ~0xffull) == a.seg_tag) {  // published from another XCD: not in this L2
            done = true;
            miss = true;
          }
        }
        if (__all(done)) break;
        if (it >= (1 << 20) || __builtin_amdgcn_s_memrealtime() - t0 > a.seg_wait) {
          miss = miss || !done;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      const unsigned long long m = __ballot(miss);
      if (p == 0) s_todo = m;
    }
    __syncthreads();
    unsigned long long todo = s_todo;
    if (todo != 0) {
      // the full pass has put only its power table (the same values) in LDS
      do {
        const int job = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int sj = REV ? nseg - 1 - job : job;
        __syncthreads();
        chunk_body<DK, DV, BN, NW, C, NT, REV, true>(a, xb + 8 * (sj - seg), smem);
      } while (todo != 0);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // states formed here are in L2 too
      __syncthreads();
    }
  };
  if constexpr (seg_early_loads(NW, NT, DK)) {
    chunk_body<DK, DV, BN, NW, C, NT, REV, false, false, false, true>(a, xb, smem, wait_entry);
  } else {
    // (a full pass with no registers to spare for its own loads across the
    // wait starts after it)
    wait_entry();
    chunk_body<DK, DV, BN, NW, C, NT, REV, false, false, false, true>(a, xb, smem);
  }
  if (wi < nseg - 1 && threadIdx.x == 0)
    __hip_atomic_store(flag + seg, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DK, int DV, int BN, int NW, int C, int NT, bool REV>
__global__ void __launch_bounds__(NW * 64) chunk_kernel_seg(ChunkArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[ChunkLds<DK, BN, C, NT, NW>::BYTES];
  __shared__ unsigned long long s_todo;
  seg_pass<DK, DV, BN, NW, C, NT, REV>(a, blockIdx.x, smem, s_todo);
}

// The backward's two transposed passes (a0 forward time, a1 reverse time),
// each split into segments, in one launch: workgroups [0, nb0) serve a0.
// nb0 is a multiple of 8, so a workgroup and the earlier segments it waits
// for still sit on one XCD.
template <int DK, int DV, int BN, int NW, int C, int NT>
__global__ void __launch_bounds__(NW * 64) chunk_kernel_seg_pair(ChunkArgs a0, ChunkArgs a1, int nb0) {
  __shared__ __attribute__((aligned(16))) char smem[ChunkLds<DK, BN, C, NT, NW>::BYTES];
  __shared__ unsigned long long s_todo;
  const int xb = blockIdx.x;
  if (xb < nb0) seg_pass<DK, DV, BN, NW, C, NT, false>(a0, xb, smem, s_todo);
  else seg_pass<DK, DV, BN, NW, C, NT, true>(a1, xb - nb0, smem, s_todo);
}

// Two independent passes of one shape in one launch, the first in forward
// time and the second in reverse time: workgroups [0, nb0) run a0, the rest
// run a1.  Each pass alone fills half the GPU.
template <int DK, int DV, int BN, int NW, int C, int NT, bool SO>
__global__ void __launch_bounds__(NW * 64) chunk_kernel_pair(ChunkArgs a0, ChunkArgs a1, int nb0) {
  __shared__ __attribute__((aligned(16))) char smem[ChunkLds<DK, BN, C, NT, NW>::BYTES];
  const int xb = blockIdx.x;
  if (xb < nb0) chunk_body<DK, DV, BN, NW, C, NT, false, SO>(a0, xb, smem);
  else chunk_body<DK, DV, BN, NW, C, NT, true, SO>(a1, xb - nb0, smem);
}

// Compute units of the device that runs stream st, looked up once per
// device (0 if that fails).
static int device_cus(hipStream_t st) {
  static std::atomic<int> cache[64];
  int dev = -1;
  const hipError_t e = st == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(st, &dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int DK, int DV, int BN, int NW, int C, int NT>
static hipError_t launch_one(const ChunkArgs& a, hipStream_t st) {
  constexpr int NBLK = DV / BN;
  const int64_t BH = a.B * a.H;
  const int64_t groups = (BH + 7) / 8;
  const int64_t nblocks = groups * 8 * NBLK * a.nseg;
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)nblocks), block(NW * 64);
  // One launch only while every workgroup can hold a compute unit of its
  // own: a workgroup that waits on a segment whose workgroup is still queued
  // behind it would hold its unit idle (two launches are faster then).
  if (a.nseg > 1 && a.seg_flag != nullptr && a.cu == nullptr && a.pool == nullptr &&
      BH * NBLK * a.nseg <= device_cus(st)) {
    if (a.reverse) hipLaunchKernelGGL((chunk_kernel_seg<DK, DV, BN, NW, C, NT, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((chunk_kernel_seg<DK, DV, BN, NW, C, NT, false>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  if (a.nseg > 1) {
    if (a.reverse) hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, false, true>), grid, block, 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.reverse) hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, true, false>), grid, block, 0, st, a);
  else if (a.cu != nullptr && a.nseg == 1)  // packed sequences (forward, no segments)
    hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, false, false, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int DK, int DV, int BN, int NW, int C, int NT>
static hipError_t launch_pair(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
  constexpr int NBLK = DV / BN;
  const int64_t BH = a0.B * a0.H;
  const int64_t groups = (BH + 7) / 8;
  const int64_t nb = groups * 8 * NBLK * a0.nseg;  // per pass (both passes share dims)
  if (nb <= 0) return hipSuccess;
  const dim3 grid((unsigned)(2 * nb)), block(NW * 64);
  if (a0.nseg > 1 && a0.seg_flag != nullptr && a1.seg_flag != nullptr &&
      2 * BH * NBLK * a0.nseg <= device_cus(st)) {  // one launch, as in launch_one
    hipLaunchKernelGGL((chunk_kernel_seg_pair<DK, DV, BN, NW, C, NT>), grid, block, 0, st, a0, a1, (int)nb);
    return hipGetLastError();
  }
  if (a0.nseg > 1) {
    hipLaunchKernelGGL((chunk_kernel_pair<DK, DV, BN, NW, C, NT, true>), grid, block, 0, st, a0, a1, (int)nb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_kernel_pair<DK, DV, BN, NW, C, NT, false>), grid, block, 0, st, a0, a1, (int)nb);
  return hipGetLastError();
}

// Forward with the output epilogue: every column of a head in one workgroup
// (the state pass of a segment split runs the same tiling without it).
template <int DK, int DV, int BN, int NW, int C, int NT>
static hipError_t launch_epi(const ChunkArgs& a, hipStream_t st) {
  static_assert(DV == BN, "the epilogue needs whole heads");
  const int64_t BH = a.B * a.H;
  const int64_t nblocks = (BH + 7) / 8 * 8 * a.nseg;
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)nblocks), block(NW * 64);
  if (a.nseg > 1) {
    hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, false, true, false>), grid, block, 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((chunk_kernel<DK, DV, BN, NW, C, NT, false, false, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

bool chunk_fused_supported(int dk, int dv, int chunk, int in_f32) {
  const bool big = dk == 96 && dv == 192, small = dk == 16 && dv == 32;
  if (!(big || small)) return false;
  if (big) return in_f32 ? (chunk == 16 || chunk == 32) : (chunk == 16 || chunk == 32 || chunk == 64);
  return chunk == 16 || chunk == 32 || chunk == 64;
}

// Tile length of the fused forward for a requested chunk: at 128 tokens its
// fp32 output staging (98 KB) does not fit beside the tiles, so bf16 inputs
// tile at 64 tokens (results equal up to rounding for every tile length).
int fused_tile(int chunk, int in_f32) { return chunk == 128 && !in_f32 ? 64 : chunk; }

int chunk_segments_fused(int64_t B, int64_t H, int64_t T, int chunk) {
  return segments_for_units(B * H, T, chunk);
}

hipError_t launch_chunk_fused(int dk, int dv, int chunk, const ChunkArgs& a, hipStream_t st) {
  if (!chunk_fused_supported(dk, dv, chunk, a.in_f32) || a.reverse) return hipErrorInvalidValue;
  if (dk == 96) {
    if (!a.in_f32) {
      switch (chunk) {
        case 16: return launch_epi<96, 192, 192, 12, 16, 1>(a, st);
        case 32: return launch_epi<96, 192, 192, 12, 32, 1>(a, st);
        default: return launch_epi<96, 192, 192, 12, 64, 1>(a, st);
      }
    }
    return chunk == 16 ? launch_epi<96, 192, 192, 12, 16, 3>(a, st) : launch_epi<96, 192, 192, 12, 32, 3>(a, st);
  }
  if (!a.in_f32) {
    switch (chunk) {
      case 16: return launch_epi<16, 32, 32, 2, 16, 1>(a, st);
      case 32: return launch_epi<16, 32, 32, 2, 32, 1>(a, st);
      default: return launch_epi<16, 32, 32, 2, 64, 1>(a, st);
    }
  }
  switch (chunk) {
    case 16: return launch_epi<16, 32, 32, 2, 16, 3>(a, st);
    case 32: return launch_epi<16, 32, 32, 2, 32, 3>(a, st);
    default: return launch_epi<16, 32, 32, 2, 64, 3>(a, st);
  }
}

int segments_for_units(int64_t units, int64_t T, int chunk) {
  constexpr int64_t kTargetUnits = 256;  // one workgroup per compute unit of an MI355X
  const int64_t nchunks = (T + chunk - 1) / chunk;
  if (units >= kTargetUnits || nchunks < 4) return 1;
  int64_t nseg = (kTargetUnits + units - 1) / units;
  if (nseg > nchunks / 2) nseg = nchunks / 2;  // at least two chunks per segment
  if (nseg > 64) nseg = 64;
  if (nseg < 2) return 1;
  // equal segments of whole chunks; drop any that would be empty
  const int64_t seg_chunks = (nchunks + nseg - 1) / nseg;
  return (int)((nchunks + seg_chunks - 1) / seg_chunks);
}

// (96, 192) with fewer than 128 (b, h) units and long segments: all 192
// columns in one 12-wave workgroup.  It runs a chunk of the whole head in
// about 1.6 times what the 6-wave tiling takes for half of it and reads k
// once, but leaves half as many workgroups per segment, so it is used where
// the split still leaves at least 8 chunks per segment (the state pass and
// fold grow with the segment count).  fp32 inputs fit its LDS up to
// 32-token chunks.
static bool wide_tiles(int dk, int dv, int chunk, int in_f32, int64_t BH, int64_t T) {
  if (!(dk == 96 && dv == 192) || BH >= 128 || chunk > (in_f32 ? 32 : 64)) return false;
  const int64_t nchunks = (T + chunk - 1) / chunk;
  return nchunks >= 8 * (int64_t)segments_for_units(BH, T, chunk);
}

// column-block width per shape and chunk (must match launch_shape)
static int block_cols(int dk, int dv, int chunk, int in_f32, int64_t BH, int64_t T) {
  if (wide_tiles(dk, dv, chunk, in_f32, BH, T)) return 192;
  if (dk == 96 && dv == 192) return 96;
  if (dk == 192 && dv == 96) return chunk <= 64 ? 96 : 48;
  return dv;  // the small shapes run all columns in one workgroup
}


int chunk_segments(int64_t B, int64_t H, int64_t T, int dk, int dv, int chunk, int in_f32) {
  const int nblk = dv / block_cols(dk, dv, chunk, in_f32, B * H, T);
  // the backward's two transposed passes share one launch when each has a
  // single column block (launch_tiles)
  return segments_for_units(B * H * nblk * ((dk > dv && nblk == 1) ? 2 : 1), T, chunk);
}

// One pass, or (a1 != null) two passes of the backward's transposed shape in
// one launch (a forward-time, a1 reverse-time).
template <int DK, int DV, int BN, int NW, int C, int NT>
static hipError_t launch_tiles(const ChunkArgs& a, const ChunkArgs* a1, hipStream_t st) {
  if constexpr (DK > DV && DV / BN == 1) {
    if (a1) return launch_pair<DK, DV, BN, NW, C, NT>(a, *a1, st);
  } else if constexpr (DK > DV) {
    // narrow column blocks already fill the GPU: the two passes run in turn
    if (a1) {
      const hipError_t e = launch_one<DK, DV, BN, NW, C, NT>(a, st);
      return e != hipSuccess ? e : launch_one<DK, DV, BN, NW, C, NT>(*a1, st);
    }
  } else {
    if (a1) return hipErrorInvalidValue;
  }
  return launch_one<DK, DV, BN, NW, C, NT>(a, st);
}

// Tile shapes per (DK, DV): BN columns per workgroup, NW waves.
template <int DK, int DV, int C, int NT>
static hipError_t launch_shape(const ChunkArgs& a, const ChunkArgs* a1, hipStream_t st) {
  if constexpr (DK == 96 && DV == 192) {
    if constexpr (C <= (NT == 1 ? 64 : 32)) {
      if (a.cu == nullptr && a.pool == nullptr && wide_tiles(DK, DV, C, a.in_f32, a.B * a.H, a.T))
        return launch_tiles<96, 192, 192, 12, C, NT>(a, a1, st);
    }
    return launch_tiles<96, 192, 96, 6, C, NT>(a, a1, st);
  }
  else if constexpr (DK == 192 && DV == 96) {
    // bf16 inputs up to 64-token chunks: all 96 columns on 12 waves, each
    // 16-column strip shared by two waves that own 96 state rows each (three
    // waves on every SIMD); fp32 inputs: 96 columns on 6 waves; 128-token
    // chunks: 48 columns on 3 waves with the wider register budget (a forward
    // of this shape; the backward tiles these passes at 64 tokens,
    // bwd_transposed_tile)
    if constexpr (C <= 64 && NT == 1) return launch_tiles<192, 96, 96, 12, C, NT>(a, a1, st);
    else if constexpr (C <= 64) return launch_tiles<192, 96, 96, 6, C, NT>(a, a1, st);
    else return launch_tiles<192, 96, 48, 3, C, NT>(a, a1, st);
  }
  else if constexpr (DK == 16 && DV == 32) return launch_tiles<16, 32, 32, 2, C, NT>(a, a1, st);
  else if constexpr (DK == 32 && DV == 16) return launch_tiles<32, 16, 16, 1, C, NT>(a, a1, st);
  else return hipErrorInvalidValue;
}

template <int DK, int DV, int NT>
static hipError_t launch_chunks(int chunk, const ChunkArgs& a, const ChunkArgs* a1, hipStream_t st) {
  switch (chunk) {
    case 16: return launch_shape<DK, DV, 16, NT>(a, a1, st);
    case 32: return launch_shape<DK, DV, 32, NT>(a, a1, st);
    case 64: return launch_shape<DK, DV, 64, NT>(a, a1, st);
    case 128: return launch_shape<DK, DV, 128, NT>(a, a1, st);
    default: return hipErrorInvalidValue;
  }
}

bool chunk_pass_supported(int dk, int dv, int chunk, int in_f32) {
  if (!(chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128)) return false;
  const bool small = (dk == 16 && dv == 32) || (dk == 32 && dv == 16);
  const bool big = (dk == 96 && dv == 192) || (dk == 192 && dv == 96);
  if (!small && !big) return false;
  if (!in_f32) return true;
  // fp32 inputs keep three bf16 planes per tile in LDS; larger tiles exceed it
  if (small || dk == 96) return chunk <= 64;
  return chunk <= 32;
}

// Tile length of the backward's transposed passes (192-row state, 96
// columns) for a requested chunk.  With bf16 inputs their 128-token tiles fit
// no layout of more than three waves per compute unit (12 waves with the row
// split need 207.5 KB of LDS; 6 waves, or 3 waves of two strips, spill
// registers), so they tile at 64 tokens; the results are equal up to rounding
// for every tile length.  Every other pass tiles at the chunk.
int bwd_transposed_tile(int chunk, int in_f32) { return chunk == 128 && !in_f32 ? 64 : chunk; }

static hipError_t launch_dispatch(int dk, int dv, int chunk, const ChunkArgs& a, const ChunkArgs* a1,
                                  hipStream_t st) {
  if (!a.in_f32) {
    if (dk == 96 && dv == 192) return launch_chunks<96, 192, 1>(chunk, a, a1, st);
    if (dk == 192 && dv == 96) return launch_chunks<192, 96, 1>(chunk, a, a1, st);
    if (dk == 16 && dv == 32) return launch_chunks<16, 32, 1>(chunk, a, a1, st);
    if (dk == 32 && dv == 16) return launch_chunks<32, 16, 1>(chunk, a, a1, st);
  } else {
    if (dk == 16 && dv == 32) {
      switch (chunk) {
        case 16: return launch_shape<16, 32, 16, 3>(a, a1, st);
        case 32: return launch_shape<16, 32, 32, 3>(a, a1, st);
        case 64: return launch_shape<16, 32, 64, 3>(a, a1, st);
        default: return hipErrorInvalidValue;
      }
    }
    if (dk == 32 && dv == 16) {
      switch (chunk) {
        case 16: return launch_shape<32, 16, 16, 3>(a, a1, st);
        case 32: return launch_shape<32, 16, 32, 3>(a, a1, st);
        case 64: return launch_shape<32, 16, 64, 3>(a, a1, st);
        default: return hipErrorInvalidValue;
      }
    }
    if (dk == 96 && dv == 192) {
      switch (chunk) {
        case 16: return launch_shape<96, 192, 16, 3>(a, a1, st);
        case 32: return launch_shape<96, 192, 32, 3>(a, a1, st);
        case 64: return launch_shape<96, 192, 64, 3>(a, a1, st);
        default: return hipErrorInvalidValue;
      }
    }
    if (dk == 192 && dv == 96) {
      switch (chunk) {
        case 16: return launch_shape<192, 96, 16, 3>(a, a1, st);
        case 32: return launch_shape<192, 96, 32, 3>(a, a1, st);
        default: return hipErrorInvalidValue;
      }
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_pass(int dk, int dv, int chunk, const ChunkArgs& a, hipStream_t st) {
  return launch_dispatch(dk, dv, chunk, a, nullptr, st);
}

hipError_t launch_chunk_pair(int dk, int dv, int chunk, const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
  if (dk <= dv || a0.reverse || !a1.reverse || a0.nseg != a1.nseg || a0.B != a1.B || a0.H != a1.H ||
      a0.T != a1.T)
    return hipErrorInvalidValue;
  return launch_dispatch(dk, dv, chunk, a0, &a1, st);
}

}  // namespace gla
