// selective_scan.hip -- gfx950 kernels for the selective (Mamba) scan.
//
// Computes, per batch b, channel d, state n (see include/sss.h):
//   Abar_t = exp(delta_t*A[d,n]),  h_t = Abar_t*h_{t-1} + delta_t*B_t[n]*x_t,
//   y_t = (sum_n C_t[n]*h_t[n] + D[d]*x_t) * silu(z_t)
// The recurrence is the selective SSM of "Selective Scan trong Mamba toi uu chuoi dai the
// nao?" (sections "Tai sao Mamba can Selective Scan?", "Selection pha vo convolution
// kernel co dinh"); the (B,L,D,N) state never leaves registers (sections "Tai sao chi
// parallel scan van chua du nhanh?" and "Kernel fusion").
//
// Mapping, chosen from measurements on MI355X (row-major (B,L,D) inputs only stream at HBM
// speed when each request covers >= 128 contiguous bytes of a row; exp issues at a quarter
// of the fp32 rate and shares the VALU with everything else):
//   * one wave = 64 consecutive channels of one batch: every load of x/delta/z and every
//     store of y is one contiguous 128-/256-byte row segment;
//   * B_t and C_t are the same for all 64 lanes, so they are read with scalar loads into
//     SGPRs and used directly as VALU operands (no LDS, no per-lane copies);
//   * each lane walks time in order with its N states in registers: per step and state
//     one exp (v_exp_f32 of delta*A*log2e), delta*x*B, the state fma and the C*h fma;
//   * time is split into S segments so that long sequences over few channels still fill
//     the GPU.  Affine steps compose associatively ("Scan bien recurrence thanh phep toan
//     co the song song hoa ra sao?": (a2,b2)(x)(a1,b1) = (a2*a1, a2*b1 + b2)), so
//       pass 1 folds each segment (but the last) into its pair (exp2(A' * sum delta), end
//              state from zero),
//       carry  composes the pairs in order from h0 into the state entering each segment,
//       pass 2 replays every segment from its entering state and writes y (and h_last).
//     With S = 1 only pass 2 runs, from h0.
#include "common.h"
#include "front.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace sss {

constexpr int kStepsPerBatch = 2;  // time steps whose x/delta/z loads are issued together
// register budget: at least this many resident waves per SIMD (512 VGPRs / waves each);
// 32 and 64 states need the larger budgets to stay spill-free
constexpr int min_waves_per_simd(int ns) { return ns >= 64 ? 1 : ns >= 32 ? 3 : 4; }
// Options that hold more per lane get larger register budgets: the exact hold keeps 1/A per
// state (2 waves per SIMD from 32 states on); channel-major tiles keep the next
// tile in flight and a tile of outputs in registers (3 waves per SIMD at 16 states with no
// other option, else 2).  (fl: bit 0 exact hold, bit 1 delta front end, bit 3 channel-major.)
constexpr int min_waves_of(int ns, int fl) {
  const int base = min_waves_per_simd(ns);
  const int cap = (fl & 8) ? (((fl & 3) != 0 || ns != 16) ? 2 : 3) : ((fl & 1) && ns >= 32) ? 2 : 4;
  return base < cap ? base : cap;
}
constexpr int kStreamPolicy = 2;    // buffer cache policy of streamed x/delta/z/y: non-temporal
constexpr int kTileBytes = 64;      // channel-major tiles: bytes of each row per tile

// Time-major rows of B and C (4, 8 or 16 states) reach the VALU from VGPRs, not SGPRs: a
// VALU instruction with a scalar operand never pairs with another wave's instruction in the
// same issue cycle, one with vector operands only does (measured on gfx950).  Each wave
// stages 1 KB of B rows (and of C rows in pass 2) in its own LDS tile, double-buffered, and
// every step reads its rows with broadcast ds_read_b128 (all lanes one address).
// (Not for channel-major rows, which stage x/delta/z in LDS instead.)
constexpr bool lds_rows(int ns, int fl) { return (fl & 8) == 0 && (ns == 4 || ns == 8 || ns == 16); }
constexpr int kRowTileBytes = 1024;  // per tensor: 256 / N steps of N fp32 states
constexpr int ilog2_const(int v) { return v <= 1 ? 0 : 1 + ilog2_const(v / 2); }
// LDS bytes per wave of the row tiles: two buffers of B (pass 1 and 3) or of B and C (pass 2,
// and pass 3 with the adjoint fold)
constexpr int row_tile_lds(int pass, bool adj = false) { return 2 * (pass == 2 || adj ? 2 : 1) * kRowTileBytes; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bit casts through by-value arguments: __builtin_bit_cast applied directly to an element of
// an ext_vector (v.y, v.z, ...) has been compiled as a cast of element 0
__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Raw buffer descriptor (gfx9 dword3) over 2^31-1 bytes from `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

constexpr int kZoh = 1, kBdl = 8;  // kFront = 2, kSoftplus = 4: common.h
// PASS 3 only: the adjoint's segment fold alongside the checkpoints (see the kernel comment)
constexpr int kAdj = 16;

// Marks running sums as needed at this point of the step.  Sums that nothing reads until the
// end of the segment are otherwise moved by the compiler to the end of the unrolled row tile,
// which keeps every step's inputs to them alive until then (hundreds of spilled registers).
template <int M>
__device__ __forceinline__ void keep_here(const float (&v)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) asm volatile("" ::"v"(v[i]));
}
__device__ __forceinline__ void keep_here(float v) { asm volatile("" ::"v"(v)); }

// Exact zero-order hold: the input coefficient expm1(u) / A with u = delta * A = arg * ln 2
// (arg = delta * A * log2 e, e2 = 2^arg).  Where |u| < 1/16 it is delta * (1 + u/2 + u^2/6 +
// u^3/24), the series of expm1(u) / u written in arg (no cancellation, and A = 0 gives delta);
// elsewhere (e2 - 1) / A with ia = 1/A.
constexpr float kZ1 = kLn2 / 2.0f, kZ2 = kLn2 * kLn2 / 6.0f, kZ3 = kLn2 * kLn2 * kLn2 / 24.0f;
constexpr float kZArg = 0.0625f / kLn2;  // |u| < 1/16 in terms of arg
__device__ __forceinline__ float zoh_coef(float arg, float e2, float dl, float ia) {
  const float q = __builtin_fmaf(arg, __builtin_fmaf(arg, __builtin_fmaf(arg, kZ3, kZ2), kZ1), 1.0f);
  const float big = __builtin_fmaf(e2, ia, -ia);
  return fabsf(arg) < kZArg ? dl * q : big;
}

struct SelSeg {
  int64_t batch, L, D, seg_len;
  int N, S, ngroups;  // ngroups = ceil(D / 64)
  int gpb;            // channel groups (waves) per workgroup, all on the same segment
  int nblk;           // workgroups per (batch, segment) = ceil(ngroups / gpb)
  int kshift, nsub;   // PASS 3: a checkpoint every 2^kshift steps, nsub per segment
  int local;          // PASS 3 with the adjoint fold: every segment from a zero state (see below)
  int vec;            // channel-major layout: 0 one step per access, 1 16-byte row pieces per
                      // lane, 2 whole tiles staged through LDS (see kTileBytes)
};

// ------------------------------------------------------------------ pass 1 / pass 2
// PASS 1 (segments 0..S-2): seg_state[s][b][n][d] = end state from zero, seg_dsum[s][b][d].
// PASS 2 (segments 0..S-1): y, and h_last from the last segment; entering state from
//         carry[s][b][n][d] (S > 1) or h0 (S == 1).
// PASS 3 (segments 0..S-1, for the backward pass): from the same entering state, the state
//         before every 2^kshift-th step into seg_state[s][b][grp][j][n][lane] (each wave's
//         checkpoints are one contiguous stream of 256-byte rows).  With kAdj it also folds
//         the segment's adjoint from a zero adjoint at its end: the backward recurrence
//         mu_{t} = a_t (mu_{t+1} + C_t dv_t) gives at the segment's first step
//         adj_mu[s][b][n][d] = sum_t P_t[n] C_t[n] dv_t with P_t = a_first ... a_t, the decays
//         this pass already forms, and dv_t = dy_t silu(z_t) (dy_t without the gate); plus the
//         segment's delta sum into seg_dsum.  (The same sum the reverse walk forms, accumulated
//         forward so that each exp serves both.)  With g.local every segment starts from a
//         zero state instead (no entering state needed, so no pass 1 before it): each
//         checkpoint then holds the state from zero plus one more row, the delta sum of the
//         segment's steps before it, and the segment's end state from zero goes to the state
//         slots passed as h_last (what pass 1 writes), for the carry.  The true state at a
//         checkpoint is that state plus exp2(A' * sum) times the segment's entering state: the
//         decays from the segment's start multiply the entering state, and their product is
//         the exponential of the summed exponents.
// FL: bit kZoh -- exact zero-order-hold input term, expm1(delta*A)/A * B instead of
//     delta * B; bits kFront / kSoftplus -- the step size is delta + bias[d], then (with
//     kSoftplus) softplus of it; bit kBdl -- x/delta/z/y channel-major (batch, dim, seqlen)
//     instead of (batch, seqlen, dim): each lane then walks its own row, loading 16 bytes
//     (8 bf16 / 4 fp32 steps) and storing 4 fp32 outputs per access where the rows are
//     16-byte aligned (g.vec), else one step per access.  B/C arrive time-major either way.
// fp32 inputs in the pass-2 form with LDS rows, and the exact hold (1/A per state) in either
// pass, keep more values in flight: 3 waves per SIMD
// (pass 3 with the adjoint fold keeps its decay products and sums: 3 as well, 2 from 32
// states on)
constexpr int min_waves_sel(int ns, int fl, bool bf16, int pass) {
  return (pass == 3 && (fl & 16) != 0)
             ? (min_waves_of(ns, fl) < (ns >= 32 ? 2 : 3) ? min_waves_of(ns, fl) : (ns >= 32 ? 2 : 3))
         : (lds_rows(ns, fl) && ((!bf16 && pass == 2) || (fl & 1) != 0) && min_waves_of(ns, fl) > 3)
             ? 3 : min_waves_of(ns, fl);
}
// Exact hold: where |delta * A| >= 2^-10 in every lane of a step (checked once per step from
// the lane's smallest |A|), (2^arg - 1) / A needs no series: its cancellation error is at most
// an ulp of 1 over |delta * A|, below 6e-5 relative there.
constexpr float kZFast = 1.0f / 1024.0f;

template <int NS, bool BF16, int PASS, bool HAS_Z, int FL>
__global__ __launch_bounds__(256, min_waves_sel(NS, FL, BF16, PASS)) void sel_seq_kernel(const void* __restrict__ x, const void* __restrict__ delta,
                                                     const float* __restrict__ A, const float* __restrict__ Bm,
                                                     const float* __restrict__ Cm, const float* __restrict__ Dsk,
                                                     const void* __restrict__ z, const float* __restrict__ h0,
                                                     const float* __restrict__ carry, float* __restrict__ y,
                                                     float* __restrict__ h_last, float* __restrict__ seg_state,
                                                     float* __restrict__ seg_dsum, const float* __restrict__ dbias,
                                                     const float* __restrict__ dy, float* __restrict__ adj_mu,
                                                     SelSeg g) {
  // Workgroup = gpb waves on adjacent channel groups and the SAME time segment, so that the
  // scalar B_t/C_t rows one wave fetches are scalar-cache hits for the others.
  const int lane = threadIdx.x & 63;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = (int)(lid % (uint32_t)g.nblk);
  lid /= (uint32_t)g.nblk;
  const int64_t b = (int64_t)(lid % (uint32_t)g.batch);
  const int s = (int)(lid / (uint32_t)g.batch);
  // wave index made provably wave-uniform, so that everything derived from it (row bases,
  // buffer descriptors) lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int grp = min(blk * g.gpb + wave, g.ngroups - 1);  // surplus waves mirror the last group
  const int64_t d0 = (int64_t)grp * 64;
  // Lanes past the last channel mirror channel D-1: same inputs, same state, same outputs,
  // so every load and store can stay unconditional (duplicate stores write equal values).
  const int64_t dc = min(d0 + lane, g.D - 1);
  const int loff = (int)(dc - d0);
  const int64_t tbeg = (int64_t)s * g.seg_len;
  const int len = (int)(min(tbeg + g.seg_len, g.L) - tbeg);  // < 2^30 (plan)
  const int N = NS;

  constexpr bool zoh = (FL & kZoh) != 0;
  constexpr bool adj = PASS == 3 && (FL & kAdj) != 0;
  float a2[NS], h[NS];
  float pp[adj ? NS : 1], mu[adj ? NS : 1];  // adjoint fold: decay product P and the sum
  // exact hold: 1/A[n]; |A| below 2^-64 (A = 0 included) gets 0 and takes the series, which
  // needs no 1/A (and covers every |delta * A| below 1/16, i.e. any delta below 2^60 there)
  float ia[zoh ? NS : 1];
  float amin = 3.402823466e+38f;  // exact hold: the lane's smallest |A[n]|
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    const float an = A[dc * N + n];
    a2[n] = fmaxf(an * kLog2e, -kFltMax);  // -inf clamped so that 0*a2 = 0
    if constexpr (zoh) {
      ia[n] = fabsf(an) >= 0x1p-64f ? 1.0f / an : 0.0f;
      amin = fminf(amin, fabsf(an));
    }
    if constexpr (adj) {
      pp[n] = 1.0f;
      mu[n] = 0.0f;
    }
    if (PASS == 1 || (adj && g.local)) {
      h[n] = 0.0f;
    } else if (g.S > 1) {
      h[n] = carry[(((int64_t)s * g.batch + b) * N + n) * g.D + dc];
    } else {
      h[n] = h0 ? h0[(b * g.D + dc) * N + n] : 0.0f;
    }
  }
  const float Dd = (PASS == 2 && Dsk != nullptr) ? Dsk[dc] : 0.0f;
  const int kmask = (1 << g.kshift) - 1;
  const float dbv = ((FL & kFront) != 0 && dbias != nullptr) ? dbias[dc] : 0.0f;
  constexpr bool has_z = (PASS == 2 || adj) && HAS_Z;
  float dsum = 0.0f;

  // Buffer descriptors based at this wave's first element of the segment: per-step offsets
  // are wave-uniform (SGPR soffset), the lane offset is a constant VGPR, so no per-load VALU
  // address arithmetic is needed.  Time-major rows: lanes are adjacent in memory and a step
  // moves by a row (the host keeps seg_len * D * 4 below 2^31); channel-major rows: each
  // lane starts its own row and a step moves by one element (the host keeps 64 * L * 4
  // below 2^31).
  constexpr bool bdl = (FL & kBdl) != 0;
  constexpr int ES = BF16 ? 2 : 4;
  const bool vec = bdl && g.vec == 1;
  // tiles only up to 16 states (the tile in flight needs 48 more registers); the host agrees
  constexpr bool kTiles = bdl && NS <= 16;
  const bool tiled = kTiles && g.vec == 2;
  const int64_t row0 = b * g.L + tbeg;
  const int64_t ebase = bdl ? (b * g.D + d0) * g.L + tbeg : row0 * g.D + d0;  // element offset
  const int rstride = bdl ? ES : (int)(g.D * ES);  // bytes between consecutive steps
  const uint32_t vo = bdl ? (uint32_t)(loff * g.L * ES) : (uint32_t)loff * ES;
  const char* const xb = (const char*)x + ebase * ES;
  const char* const db = (const char*)delta + ebase * ES;
  const char* const zb = has_z ? (const char*)z + ebase * ES : (const char*)x;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xb);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(db);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(zb);
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(PASS == 2 ? (const char*)(y + ebase) : (const char*)x);
  const __amdgpu_buffer_rsrc_t rdy = make_rsrc(adj ? (const char*)(dy + ebase) : (const char*)x);
  const int ystride = bdl ? 4 : (int)(g.D * 4);
  const uint32_t yvo = bdl ? (uint32_t)(loff * g.L * 4) : (uint32_t)loff * 4;
  // channel-major output goes through the caches so that the row pieces of consecutive
  // stores merge into whole lines before they reach HBM
  constexpr int kYPolicy = bdl ? 0 : kStreamPolicy;
  constexpr int kInPolicy = bdl ? 0 : kStreamPolicy;
  const float* Br = Bm + row0 * N;
  const float* Cr = Cm + row0 * N;

  // B/C row tiles (time-major, 4/8/16 states): tile j holds segment steps [j*kRT, (j+1)*kRT),
  // one 16-byte piece per lane; loads past the end of the sequence go through descriptors
  // whose range stops there (the hardware returns zeros for them).  Each piece covers whole
  // rows or whole quarters of a row, so the range check never splits a row.
  constexpr bool kRows = lds_rows(NS, FL);
  constexpr int kRT = kRows ? kRowTileBytes / (4 * NS) : 1;  // steps per row tile
  constexpr int kRTShift = ilog2_const(kRT);
  constexpr int kRowTensors = PASS == 2 || adj ? 2 : 1;
  extern __shared__ uint32_t sss_lds[];  // dynamic LDS: the row tiles or the channel-major tiles
  float* const lrows = reinterpret_cast<float*>(sss_lds) + wave * (row_tile_lds(PASS, adj) / 4);  // [buf][tensor][256]
  const int64_t row_bytes_rem = (g.L - tbeg) * N * 4;  // rows of B/C from this segment to the end
  const uint32_t row_bytes_left = row_bytes_rem < 0x7FFFFFF0 ? (uint32_t)row_bytes_rem : 0x7FFFFFF0u;
  const __amdgpu_buffer_rsrc_t rrb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Br), 0, (int)row_bytes_left, 0x00020000);
  const __amdgpu_buffer_rsrc_t rrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Cr), 0, (int)row_bytes_left, 0x00020000);
  u32x4 grb = {0u, 0u, 0u, 0u}, grc = {0u, 0u, 0u, 0u};
  auto rows_load = [&](int j) {  // row tile j -> registers
    if constexpr (kRows) {
      grb = __builtin_amdgcn_raw_buffer_load_b128(rrb, lane * 16, j * kRowTileBytes, 0);
      if constexpr (kRowTensors == 2) grc = __builtin_amdgcn_raw_buffer_load_b128(rrc, lane * 16, j * kRowTileBytes, 0);
    }
  };
  auto rows_store = [&](int buf) {  // registers -> LDS buffer buf
    if constexpr (kRows) {
      *reinterpret_cast<u32x4*>(lrows + buf * (kRowTensors * 256) + lane * 4) = grb;
      if constexpr (kRowTensors == 2) *reinterpret_cast<u32x4*>(lrows + buf * (kRowTensors * 256) + 256 + lane * 4) = grc;
    }
  };

  // steps per load batch: 2 time-major steps, or one 16-byte piece of a channel-major row
  constexpr int U = bdl ? 16 / ES : kStepsPerBatch;
  constexpr int QW = bdl ? 4 : U;  // raw dwords per tensor and batch
  constexpr int TT = kTileBytes / ES;  // channel-major tile: steps per tile
  // raw loaded values (bf16 bits or fp32 bits) are widened only when used, so that the
  // loads of the next batch stay in flight while the current batch is computed
  uint32_t xq[2][QW], dq[2][QW], zq[2][QW];
  uint32_t gq_dy[2][adj ? QW : 1];  // adjoint fold: dy bits (time-major only)
  // channel-major: outputs stored together -- a batch, or a whole tile (a full row piece
  // of y per lane, written by consecutive stores) when tiles are used
  constexpr int YT = kTileBytes / ES;  // tiled: y steps per store group (a whole tile)
  float yb[bdl ? (NS <= 16 ? YT : U) : 1];
  auto ld = [vo](__amdgpu_buffer_rsrc_t r, int soff) -> uint32_t {
    if (BF16) return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)vo, soff, kInPolicy);
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, soff, kInPolicy);
  };
  // one 16-byte piece of the lane's row
  auto ld4 = [&](uint32_t (&q)[QW], __amdgpu_buffer_rsrc_t r, int soff) {
    if constexpr (QW == 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, soff, kInPolicy);
      q[0] = v.x;
      q[1] = v.y;
      q[2] = v.z;
      q[3] = v.w;
    }
  };
  auto wid = [](uint32_t v) -> float { return BF16 ? __builtin_bit_cast(float, v << 16) : __builtin_bit_cast(float, v); };
  // step I of a batch
  auto val = [&](const uint32_t (&q)[QW], int i) -> float {
    if constexpr (!bdl) return wid(q[i]);
    if constexpr (BF16) return u32_as_f32((i & 1) ? (q[i >> 1] & 0xFFFF0000u) : (q[i >> 1] << 16));
    return u32_as_f32(q[i]);
  };
  // channel-major, unaligned rows: one step per access, packed like a 16-byte piece
  auto ld_steps = [&](uint32_t (&q)[QW], __amdgpu_buffer_rsrc_t r, int t0) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const uint32_t v = ld(r, min(t0 + i, len - 1) * ES);
      if (BF16) q[i >> 1] = (i & 1) ? (q[i >> 1] | (v << 16)) : v;
      else q[i] = v;
    }
  };
  // Channel-major rows whose length is a multiple of the tile: the wave's 64 rows are
  // staged kTileBytes at a time.  Each load instruction takes 16 rows x kTileBytes (four
  // lanes per row, so rows are read in whole 64-byte pieces), the pieces go to this wave's
  // LDS tile, and each lane then reads its own row 16 bytes per batch.  The next tile's
  // loads are in flight (gq) while the current tile is computed.  LDS rows are 64 bytes
  // with the 16-byte chunks xor-swizzled by row (by row / 4: four rows share one 256-byte
  // bank line), so that the lanes' 16-byte reads of one batch fall in distinct banks.
  constexpr int kNT = has_z ? 3 : 2;  // tensors staged: x, delta (, z)
  constexpr int kPieces = 4;          // 16-byte pieces per lane, tensor and tile
  // channel-major tiles in the same dynamic LDS: [wave][tensor][64 rows][16 dwords]
  uint32_t* const ltile = sss_lds + wave * (kNT * 64 * 16);
  uint32_t gq[kNT][kPieces][4];
  uint32_t gvo[kPieces];  // lane's byte offset of piece i: row 16 i + lane / 4, chunk lane % 4
  int gchunk[kPieces];    // LDS dword offset of that piece within a tensor tile
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int r = 16 * i + (lane >> 2), c = lane & 3;
    const int rr = (int)(min(d0 + r, g.D - 1) - d0);  // rows past D-1 repeat the last row
    gvo[i] = (uint32_t)(rr * g.L * ES + c * 16);
    gchunk[i] = r * 16 + ((c ^ ((r >> 2) & 3)) * 4);
  }
  const int lrow = loff * 16;
  const int lswz = (loff >> 2) & 3;
  // tile starting at segment step t0.  The loop stays branch-free: the two loads past the
  // segment's end (their tiles are never read) go through descriptors of zero bytes, so the
  // hardware's range check returns zeros without touching memory.
  // Pass 2 keeps the tile lines cached (the second half of each line is read a tile later;
  // measured: 1.27 -> 1.21 ms on the long layer), pass 1 streams them (cached was slower).
  constexpr int kTilePolicy = PASS == 2 ? 0 : kStreamPolicy;
  auto tile_load = [&](int t0) {
    const bool inside = t0 < len;  // wave-uniform
    const int so = inside ? t0 * ES : 0;
    const int nrec = inside ? 0x7FFFFFFF : 0;
    const __amdgpu_buffer_rsrc_t tx = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(xb), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t td = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(db), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t tz = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(zb), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int vo_ = (int)gvo[i];
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(tx, vo_, so, kTilePolicy);
      const u32x4 bq = __builtin_amdgcn_raw_buffer_load_b128(td, vo_, so, kTilePolicy);
      gq[0][i][0] = a.x; gq[0][i][1] = a.y; gq[0][i][2] = a.z; gq[0][i][3] = a.w;
      gq[1][i][0] = bq.x; gq[1][i][1] = bq.y; gq[1][i][2] = bq.z; gq[1][i][3] = bq.w;
      if constexpr (kNT == 3) {
        const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(tz, vo_, so, kTilePolicy);
        gq[2][i][0] = c.x; gq[2][i][1] = c.y; gq[2][i][2] = c.z; gq[2][i][3] = c.w;
      }
    }
  };
  auto tile_store = [&]() {  // the tile in flight -> this wave's LDS tile
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const u32x4 v = {gq[t][i][0], gq[t][i][1], gq[t][i][2], gq[t][i][3]};
        *reinterpret_cast<u32x4*>(ltile + t * (64 * 16) + gchunk[i]) = v;
      }
    }
  };
  auto tile_read = [&](uint32_t (&q)[QW], int t, int kb) {  // batch kb of the lane's row
    if constexpr (QW == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(ltile + t * (64 * 16) + lrow + ((kb ^ lswz) * 4));
      q[0] = v.x;
      q[1] = v.y;
      q[2] = v.z;
      q[3] = v.w;
    }
  };
  if (tiled) {
    tile_load(0);
    tile_store();
    tile_load(TT);
  }
  // PASS 3: the checkpoint before segment step t, [s][b][grp][j][row][lane] with NS + 1
  // rows of 256 bytes per checkpoint (the states, then the delta sum of the steps before it
  // when every segment starts from zero)
  auto ck_store = [&](int t) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(
        seg_state + ((((int64_t)s * g.batch + b) * g.ngroups + grp) * g.nsub + (t >> g.kshift)) * (N + 1) * 64);
#pragma unroll
    for (int n = 0; n < NS; ++n)
      __builtin_amdgcn_raw_buffer_store_b32(f32_as_u32(h[n]), rk, lane * 4, n * 256, kStreamPolicy);
    if (adj && g.local) __builtin_amdgcn_raw_buffer_store_b32(f32_as_u32(dsum), rk, lane * 4, N * 256, kStreamPolicy);
  };
#define SSS_LOAD_BATCH(SLOT, T0)                                                 \
  do {                                                                           \
    if constexpr (!bdl) {                                                        \
      _Pragma("unroll") for (int i_ = 0; i_ < U; ++i_) {                         \
        const int t_ = min((T0) + i_, len - 1); /* clamped, unused */            \
        xq[SLOT][i_] = ld(rx, t_ * rstride);                                     \
        dq[SLOT][i_] = ld(rd, t_ * rstride);                                     \
        if (has_z) zq[SLOT][i_] = ld(rz, t_ * rstride);                          \
        if constexpr (adj)                                                       \
          gq_dy[SLOT][i_] = __builtin_amdgcn_raw_buffer_load_b32(rdy, (int)yvo, t_ * ystride, kInPolicy); \
      }                                                                          \
    } else if (vec) { /* len is a multiple of U: the clamp stays aligned */      \
      const int so_ = min((T0), len - U) * ES;                                   \
      ld4(xq[SLOT], rx, so_);                                                    \
      ld4(dq[SLOT], rd, so_);                                                    \
      if (has_z) ld4(zq[SLOT], rz, so_);                                         \
    } else {                                                                     \
      ld_steps(xq[SLOT], rx, (T0));                                              \
      ld_steps(dq[SLOT], rd, (T0));                                              \
      if (has_z) ld_steps(zq[SLOT], rz, (T0));                                   \
    }                                                                            \
  } while (0)

  // one step at segment-relative time T from register slot (SLOT, I); B_t / C_t rows are
  // wave-uniform and come through scalar loads
#define SSS_STEP_BC(SLOT, I, T, YI, BT, CT)                                      \
  do {                                                                           \
    const float* Bt = (BT);                                                      \
    const float* Ct = (CT);                                                      \
    if (PASS == 3 && ((T) & kmask) == 0) ck_store(T);                            \
    const float xv = val(xq[SLOT], I);                                           \
    const float dl = step_size<FL>(val(dq[SLOT], I), dbv);                       \
    const float dx = dl * xv;                                                    \
    float y0 = Dd * xv, y1 = 0.0f;                                               \
    float dvv = 0.0f; /* adjoint fold: dy silu(z) */                             \
    if constexpr (adj) {                                                         \
      dvv = u32_as_f32(gq_dy[SLOT][I]);                         \
      if (has_z) dvv *= silu(val(zq[SLOT], I));                                  \
    }                                                                            \
    /* states in groups of 4: the arguments, the exps at a raised wave priority,   \
       then the updates (as the row-tile step); the rows are read ahead of them,   \
       all at once up to 32 states, a group at a time above (64 states' rows of B  \
       and C would not fit the scalar registers) */                                \
    constexpr int GB_ = NS < 4 ? NS : 4;                                         \
    constexpr int RA_ = NS <= 32 ? NS : GB_;                                     \
    float bt_[RA_], ct_[(PASS == 2 || adj) ? RA_ : 1];                           \
    auto rows_ahead_ = [&](int r0) {                                             \
      _Pragma("unroll") for (int r = 0; r < RA_; ++r) {                          \
        bt_[r] = Bt[r0 + r];                                                     \
        if constexpr (PASS == 2 || adj) ct_[r] = Ct[r0 + r];                     \
      }                                                                          \
    };                                                                           \
    if constexpr (RA_ == NS) rows_ahead_(0);                                     \
    _Pragma("unroll") for (int n0 = 0; n0 < NS; n0 += GB_) {                     \
    if constexpr (RA_ != NS) rows_ahead_(n0);                                    \
    constexpr int RB_ = RA_ == NS ? 1 : 0; /* row index base: n, or n - n0 */    \
    float args_[GB_], abs_[GB_];                                                 \
    _Pragma("unroll") for (int k = 0; k < GB_; ++k) args_[k] = dl * a2[n0 + k];  \
    __builtin_amdgcn_sched_barrier(0x14);                                        \
    __builtin_amdgcn_s_setprio(2);                                               \
    _Pragma("unroll") for (int k = 0; k < GB_; ++k) abs_[k] = fast_exp2(args_[k]); \
    __builtin_amdgcn_s_setprio(0);                                               \
    __builtin_amdgcn_sched_barrier(0x14);                                        \
    _Pragma("unroll") for (int k = 0; k < GB_; ++k) {                            \
      const int n = n0 + k;                                                      \
      const int r_ = RB_ ? n : k; /* the state's row entry */                    \
      const float arg = args_[k];                                                \
      const float ab = abs_[k];                                                  \
      if constexpr (adj) {                                                       \
        pp[n] *= ab;                                                             \
        mu[n] = __builtin_fmaf(pp[n], ct_[r_] * dvv, mu[n]);                     \
      }                                                                          \
      if constexpr (zoh) {                                                       \
        const float cf = zoh_coef(arg, ab, dl, ia[n]);                          \
        h[n] = __builtin_fmaf(ab, h[n], cf * (xv * bt_[r_]));                    \
      } else {                                                                   \
        h[n] = __builtin_fmaf(ab, h[n], dx * bt_[r_]);                           \
      }                                                                          \
      if constexpr (PASS == 2) {                                                 \
        if (n & 1) y1 = __builtin_fmaf(ct_[r_], h[n], y1);                       \
        else y0 = __builtin_fmaf(ct_[r_], h[n], y0);                             \
      }                                                                          \
    }                                                                            \
    __builtin_amdgcn_sched_barrier(0x14);                                        \
    }                                                                            \
    if (PASS == 1 || adj) {                                                      \
      dsum += dl;                                                                \
      if constexpr (adj) keep_here(mu);                                          \
      keep_here(dsum);                                                           \
    } else if (PASS == 2) {                                                      \
      float out = y0 + y1;                                                       \
      if (has_z) out *= silu(val(zq[SLOT], I));                                  \
      if constexpr (bdl) {                                                       \
        yb[(YI)] = out;                                                          \
      } else {                                                                   \
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), ry, (int)yvo, \
                                              (T) * ystride, kYPolicy);          \
      }                                                                          \
    }                                                                            \
  } while (0)

#define SSS_STEP_Y(SLOT, I, T, YI) SSS_STEP_BC(SLOT, I, T, YI, Br + (T) * N, Cr + (T) * N)
#define SSS_STEP(SLOT, I, T) SSS_STEP_Y(SLOT, I, T, I)

  // channel-major: the batch's outputs, steps T0 .. T0+CNT-1
#define SSS_STORE_BATCH(T0, CNT)                                                 \
  do {                                                                           \
    if constexpr (bdl && PASS == 2) {                                            \
      if (vec || tiled) {                                                        \
        _Pragma("unroll") for (int j_ = 0; j_ < U; j_ += 4) {                    \
          const u32x4 o_ = {f32_as_u32(yb[j_]), f32_as_u32(yb[j_ + 1]), f32_as_u32(yb[j_ + 2]), \
                            f32_as_u32(yb[j_ + 3])};                             \
          __builtin_amdgcn_raw_buffer_store_b128(o_, ry, (int)yvo, ((T0) + j_) * 4, kYPolicy); \
        }                                                                        \
      } else {                                                                   \
        _Pragma("unroll") for (int j_ = 0; j_ < U; ++j_)                         \
          if (j_ < (CNT))                                                        \
            __builtin_amdgcn_raw_buffer_store_b32(f32_as_u32(yb[j_]), ry, (int)yvo, ((T0) + j_) * 4, kYPolicy); \
      }                                                                          \
    }                                                                            \
  } while (0)

  // One step at segment-relative time t with B/C rows from the LDS tile, each group of
  // states in three phases separated by scheduling barriers that only memory and scalar
  // instructions may cross: the exponent arguments, the exps, then the multiplies and fmas
  // of the update and read-out.  Grouped like this, the VGPR-only instructions of one wave meet those of
  // another more often and issue in pairs (measured: the per-state cost of the pass-2
  // pattern drops from ~24 to ~21 clocks).
  // The exp phase runs at a raised wave priority: a wave that reaches its exps issues them
  // ahead of the other waves' multiplies and fmas, which then meet in their own phases and
  // issue in pairs more often (measured on the phased step alone: 337 -> 301 clocks per
  // 16-state step at four waves per SIMD; the long layer's call 1.65-1.66 -> 1.56 ms).
  constexpr bool kExpPrio = true;
  auto lstep = [&](const uint32_t (&xs)[QW], const uint32_t (&dqs)[QW], const uint32_t (&zs)[QW],
                   const uint32_t (&dys)[adj ? QW : 1], int i, int t) {
    if constexpr (kRows) {
      const float* brow = lrows + ((t >> kRTShift) & 1) * (kRowTensors * 256) + (t & (kRT - 1)) * NS;
      if (PASS == 3 && (t & kmask) == 0) ck_store(t);
      const float xv = val(xs, i);
      const float dl = step_size<FL>(val(dqs, i), dbv);
      const float dx = dl * xv;
      float y0 = Dd * xv, y1 = 0.0f;
      float dvv = 0.0f;  // adjoint fold: dy silu(z)
      if constexpr (adj) {
        dvv = u32_as_f32(dys[i]);
        if constexpr (has_z) dvv *= silu(val(zs, i));
      }
      // states in groups of GS (the phases of one group hold GS arguments, GS decays and GS
      // rows of B and C in registers)
      constexpr int GS = NS < 8 ? NS : (BF16 && PASS != 2 && !zoh && !adj ? 8 : 4);  // pass 2, fp32 inputs, exact hold, adjoint: more registers
      constexpr bool kC = PASS == 2 || adj;  // C rows used
#pragma unroll
      for (int n0 = 0; n0 < NS; n0 += GS) {
        float bq[GS], cq[kC ? GS : 1];
#pragma unroll
        for (int q = 0; q < GS / 4; ++q) {
          const float4 v = reinterpret_cast<const float4*>(brow + n0)[q];
          bq[4 * q] = v.x; bq[4 * q + 1] = v.y; bq[4 * q + 2] = v.z; bq[4 * q + 3] = v.w;
          if constexpr (kC) {
            const float4 c = reinterpret_cast<const float4*>(brow + 256 + n0)[q];
            cq[4 * q] = c.x; cq[4 * q + 1] = c.y; cq[4 * q + 2] = c.z; cq[4 * q + 3] = c.w;
          }
        }
        float arg[GS], ab[GS];
#pragma unroll
        for (int k = 0; k < GS; ++k) arg[k] = dl * a2[n0 + k];
        __builtin_amdgcn_sched_barrier(0x14);
        if constexpr (kExpPrio) __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int k = 0; k < GS; ++k) ab[k] = fast_exp2(arg[k]);
        if constexpr (kExpPrio) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0x14);
#pragma unroll
        for (int k = 0; k < GS; ++k) {
          const int n = n0 + k;
          if constexpr (zoh) {  // direct form: (2^arg - 1) / A * x B = fma(2^arg, w, -w), w = x B / A
            const float w = ia[n] * (xv * bq[k]);
            h[n] = __builtin_fmaf(ab[k], h[n], __builtin_fmaf(ab[k], w, -w));
          } else {
            h[n] = __builtin_fmaf(ab[k], h[n], dx * bq[k]);
          }
          if constexpr (PASS == 2) {
            if (n & 1) y1 = __builtin_fmaf(cq[k], h[n], y1);
            else y0 = __builtin_fmaf(cq[k], h[n], y0);
          }
          if constexpr (adj) {
            pp[n] *= ab[k];
            mu[n] = __builtin_fmaf(pp[n], cq[k] * dvv, mu[n]);
          }
        }
        __builtin_amdgcn_sched_barrier(0x14);
      }
      if constexpr (zoh) {
        // Exact hold, a step where some lane has |delta * A| below 2^-10 for one of its states:
        // the direct form above loses accuracy to cancellation there, so each state gets the
        // difference between the exact coefficient (series for small arguments) and the
        // direct one added afterwards.  The direct term is recomputed here by the same
        // operations, from a copy of the step size that the compiler cannot see through, so
        // that none of it is kept live from the common path (which needs no branch join).
        if (__builtin_amdgcn_ballot_w64(fabsf(dl) * amin >= kZFast) != __builtin_amdgcn_read_exec()) {
          float dls = dl;
          asm volatile("; exact hold, series correction" : "+v"(dls));
#pragma unroll
          for (int n0 = 0; n0 < NS; n0 += 4) {
            const float4 v = reinterpret_cast<const float4*>(brow + n0)[0];
            const float bq[4] = {v.x, v.y, v.z, v.w};
            float cq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (PASS == 2) {
              const float4 c = reinterpret_cast<const float4*>(brow + 256 + n0)[0];
              cq[0] = c.x; cq[1] = c.y; cq[2] = c.z; cq[3] = c.w;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int n = n0 + k;
              const float arg = dls * a2[n];
              const float e = fast_exp2(arg);
              const float xb = xv * bq[k];
              const float w = ia[n] * xb;
              const float d = zoh_coef(arg, e, dls, ia[n]) * xb - __builtin_fmaf(e, w, -w);
              h[n] += d;
              if constexpr (PASS == 2) y0 = __builtin_fmaf(cq[k], d, y0);
            }
          }
        }
      }
      if constexpr (PASS == 1 || adj) {
        dsum += dl;
        if constexpr (adj) keep_here(mu);
        keep_here(dsum);
      } else if constexpr (PASS == 2) {
        float out = y0 + y1;
        if constexpr (has_z) out *= silu(val(zs, i));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, out), ry, (int)yvo, t * ystride, kYPolicy);
      }
    }
  };

  int t0 = 0;
  if constexpr (kTiles) {
    // Channel-major tiles (len is a multiple of the tile): one tile per iteration, its
    // batches read from LDS one ahead; the next tile (in flight since the previous
    // iteration) is stored to LDS once the current one is consumed, and the one after it
    // loaded.  y is kept for the whole tile (a 128-byte line of each row in bf16, half a
    // line in fp32) and leaves through the consumed LDS tile: each lane writes its row,
    // then every store instruction takes whole row pieces (YC lanes per row, 64 / YC rows),
    // so that each line is written by one instruction instead of a 16-byte piece at a time
    // by YC of them.  LDS y rows hold YC 16-byte chunks, xor-swizzled by row so that both
    // the row-wise writes and the piece-wise reads fall in distinct banks.
    constexpr int kB = TT / U;  // batches per tile: 4
    static_assert(kB == 4 && YT == TT, "tile layout");
    constexpr int YC = YT / 4;                 // 16-byte chunks of y per row and tile: 8 or 4
    constexpr int YRS = 16 / YC;               // rows per 256 bytes of LDS: 2 or 4
    static_assert(YC <= 4 * kNT, "the y tile fits in the input tile");
    if (tiled) {
      tile_read(xq[0], 0, 0);
      tile_read(dq[0], 1, 0);
      if constexpr (has_z) tile_read(zq[0], 2, 0);
    }
#define SSS_TILE_READ(SLOT, KB)                                                  \
  do {                                                                           \
    tile_read(xq[SLOT], 0, KB);                                                  \
    tile_read(dq[SLOT], 1, KB);                                                  \
    if constexpr (has_z) tile_read(zq[SLOT], 2, KB);                             \
  } while (0)
    // the tile's outputs (steps TY .. TY+YT-1) through the consumed LDS tile
    auto y_tile = [&](int ty) {
      if constexpr (PASS == 2) {
        uint32_t* const ly = ltile;
        const int wrow = lane * (YC * 4);
        const int wswz = (lane / YRS) & (YC - 1);
#pragma unroll
        for (int c = 0; c < YC; ++c) {
          const u32x4 o = {f32_as_u32(yb[4 * c]), f32_as_u32(yb[4 * c + 1]), f32_as_u32(yb[4 * c + 2]),
                           f32_as_u32(yb[4 * c + 3])};
          *reinterpret_cast<u32x4*>(ly + wrow + ((c ^ wswz) * 4)) = o;
        }
        const int pc = lane % YC;  // the lane's chunk of each row piece it stores
#pragma unroll
        for (int k = 0; k < YC; ++k) {
          const int r = k * (64 / YC) + lane / YC;  // row of this store
          const u32x4 o = *reinterpret_cast<const u32x4*>(ly + r * (YC * 4) + ((pc ^ ((r / YRS) & (YC - 1))) * 4));
          // rows past the last channel hold channel D-1's values: store them there again
          const int rr = (int)min((int64_t)r, g.D - 1 - d0);
          __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)((uint32_t)rr * (uint32_t)g.L * 4u + pc * 16), ty * 4,
                                                 kYPolicy);
        }
      }
    };
    // Pass 2 takes its B_t / C_t rows one step ahead: each step first waits for its own rows
    // (and for the LDS reads issued a step earlier), then issues the next step's row loads and
    // the batch's LDS read, so that the scalar loads have a whole step to arrive instead of
    // the few instructions the compiler leaves between a load and its first use.  (With
    // three resident waves per SIMD, the fewest of any forward kernel, those waits were
    // not hidden.)
    float bq[2][NS], cq[2][NS];
    auto bc_load = [&](int slot, int t) {
      const float* bp = Br + t * N;
      const float* cp = Cr + t * N;
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        bq[slot][n] = bp[n];
        if constexpr (PASS == 2) cq[slot][n] = cp[n];
      }
    };
#define SSS_TSTEP(SLOT, I, T, YI, ACTION)                                        \
  do {                                                                           \
    if constexpr (PASS == 2) {                                                   \
      __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */                       \
      __builtin_amdgcn_sched_barrier(0);                                         \
      bc_load(((YI) & 1) ^ 1, min((T) + 1, len - 1));                            \
      ACTION;                                                                    \
      __builtin_amdgcn_sched_barrier(0);                                         \
      SSS_STEP_BC(SLOT, I, T, YI, bq[(YI) & 1], cq[(YI) & 1]);                   \
    } else {                                                                     \
      ACTION;                                                                    \
      SSS_STEP_Y(SLOT, I, T, YI);                                                \
    }                                                                            \
  } while (0)
    if (PASS == 2 && tiled) bc_load(0, 0);
    for (; tiled && t0 < len; t0 += TT) {
      SSS_TSTEP(0, 0, t0, 0, SSS_TILE_READ(1, 1));
#pragma unroll
      for (int i = 1; i < U; ++i) SSS_TSTEP(0, i, t0 + i, i, );
      SSS_TSTEP(1, 0, t0 + U, U, SSS_TILE_READ(0, 2));
#pragma unroll
      for (int i = 1; i < U; ++i) SSS_TSTEP(1, i, t0 + U + i, U + i, );
      SSS_TSTEP(0, 0, t0 + 2 * U, 2 * U, SSS_TILE_READ(1, 3));
#pragma unroll
      for (int i = 1; i < U; ++i) SSS_TSTEP(0, i, t0 + 2 * U + i, 2 * U + i, );
      if constexpr (PASS == 2) {
#pragma unroll
        for (int i = 0; i < U; ++i) SSS_TSTEP(1, i, t0 + 3 * U + i, 3 * U + i, );
        y_tile(t0);              // the LDS tile is consumed: stage y through it
        tile_store();            // the next tile, loaded during the previous iteration
        tile_load(t0 + 2 * TT);  // the one after it
        SSS_TILE_READ(0, 0);
      } else {
        tile_store();
        tile_load(t0 + 2 * TT);
        SSS_TILE_READ(0, 0);
#pragma unroll
        for (int i = 0; i < U; ++i) SSS_TSTEP(1, i, t0 + 3 * U + i, 3 * U + i, );
      }
    }
#undef SSS_TSTEP
#undef SSS_TILE_READ
  }
  if (!tiled) SSS_LOAD_BATCH(0, 0);
  if constexpr (kRows) {
    // row tile 0 in LDS, tile 1 in flight
    rows_load(0);
    rows_store(0);
    rows_load(1);
    // whole row tiles: kRT steps per iteration, then the next tile (loaded a whole tile
    // earlier) goes to the other buffer and the one after it is loaded
    for (; t0 + kRT <= len; t0 += kRT) {
#pragma unroll
      for (int q = 0; q < kRT; q += 2 * U) {
        SSS_LOAD_BATCH(1, t0 + q + U);
#pragma unroll
        for (int i = 0; i < U; ++i) lstep(xq[0], dq[0], zq[0], gq_dy[0], i, t0 + q + i);
        SSS_LOAD_BATCH(0, t0 + q + 2 * U);
#pragma unroll
        for (int i = 0; i < U; ++i) lstep(xq[1], dq[1], zq[1], gq_dy[1], i, t0 + q + U + i);
      }
      rows_store(((t0 >> kRTShift) + 1) & 1);
      rows_load((t0 >> kRTShift) + 2);
    }
    // fewer than kRT steps left, all in the tile now in LDS
    for (; t0 + 2 * U <= len; t0 += 2 * U) {
      SSS_LOAD_BATCH(1, t0 + U);
#pragma unroll
      for (int i = 0; i < U; ++i) lstep(xq[0], dq[0], zq[0], gq_dy[0], i, t0 + i);
      SSS_LOAD_BATCH(0, t0 + 2 * U);
#pragma unroll
      for (int i = 0; i < U; ++i) lstep(xq[1], dq[1], zq[1], gq_dy[1], i, t0 + U + i);
    }
    if (t0 < len) {
      SSS_LOAD_BATCH(1, t0 + U);
#pragma unroll
      for (int i = 0; i < U; ++i)
        if (t0 + i < len) lstep(xq[0], dq[0], zq[0], gq_dy[0], i, t0 + i);
      if (t0 + U < len) {
#pragma unroll
        for (int i = 0; i < U; ++i)
          if (t0 + U + i < len) lstep(xq[1], dq[1], zq[1], gq_dy[1], i, t0 + U + i);
      }
    }
    t0 = len;
  }
  // full blocks of 2U steps: straight-line code, no per-step branches
  for (; t0 + 2 * U <= len; t0 += 2 * U) {
    SSS_LOAD_BATCH(1, t0 + U);
#pragma unroll
    for (int i = 0; i < U; ++i) SSS_STEP(0, i, t0 + i);
    SSS_STORE_BATCH(t0, U);
    SSS_LOAD_BATCH(0, t0 + 2 * U);
#pragma unroll
    for (int i = 0; i < U; ++i) SSS_STEP(1, i, t0 + U + i);
    SSS_STORE_BATCH(t0 + U, U);
  }
  // ragged tail (< 2U steps): slot 0 already holds steps t0 .. t0+U-1
  if (t0 < len) {
    SSS_LOAD_BATCH(1, t0 + U);
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (t0 + i < len) SSS_STEP(0, i, t0 + i);
    SSS_STORE_BATCH(t0, min(U, len - t0));
    if (t0 + U < len) {
#pragma unroll
      for (int i = 0; i < U; ++i)
        if (t0 + U + i < len) SSS_STEP(1, i, t0 + U + i);
      SSS_STORE_BATCH(t0 + U, len - t0 - U);
    }
  }
#undef SSS_LOAD_BATCH
#undef SSS_STEP
#undef SSS_STEP_Y
#undef SSS_STEP_BC
#undef SSS_STORE_BATCH

  if (PASS == 1) {
    if (lane == 0 || d0 + lane < g.D) seg_dsum[((int64_t)s * g.batch + b) * g.D + dc] = dsum;
#pragma unroll
    for (int n = 0; n < NS; ++n) seg_state[(((int64_t)s * g.batch + b) * N + n) * g.D + dc] = h[n];
  } else if (adj) {
    if (lane == 0 || d0 + lane < g.D) seg_dsum[((int64_t)s * g.batch + b) * g.D + dc] = dsum;
#pragma unroll
    for (int n = 0; n < NS; ++n) adj_mu[(((int64_t)s * g.batch + b) * N + n) * g.D + dc] = mu[n];
    if (g.local && s < g.S - 1) {  // end state from zero, as pass 1 leaves it for the carry
#pragma unroll
      for (int n = 0; n < NS; ++n) h_last[(((int64_t)s * g.batch + b) * N + n) * g.D + dc] = h[n];
    }
  } else if (PASS == 2 && h_last != nullptr && s == g.S - 1) {
#pragma unroll
    for (int n = 0; n < NS; ++n) h_last[(b * g.D + dc) * N + n] = h[n];
  }
}

// ------------------------------------------------------------------ carry between segments
// One thread per (b, n, d), in place over the segment states: slot s holds the end state
// of segment s from zero on entry and the state entering segment s on exit,
//   carry[0] = h0,  carry[s+1] = exp2(A' * dsum_s) * carry[s] + state_s.
// Loads of a batch of segments are issued before the serial fma chain consumes them.
constexpr int kCarryBatch = 8;

static __global__ __launch_bounds__(256) void sel_carry_kernel(const float* __restrict__ A, const float* __restrict__ h0,
                                                        float* slots, const float* __restrict__ seg_dsum, SelSeg g) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_b = (int64_t)g.N * g.D;
  if (idx >= g.batch * per_b) return;
  const int64_t b = idx / per_b;
  const int64_t rem = idx - b * per_b;
  const int64_t n = rem / g.D, d = rem - n * g.D;
  const float a2 = fmaxf(A[d * g.N + n] * kLog2e, -kFltMax);
  float h = h0 ? h0[(b * g.D + d) * g.N + n] : 0.0f;
  const int64_t sstride = g.batch * per_b, dstride = g.batch * g.D;
  float* slot = slots + b * per_b + rem;              // [s][b][n][d]
  const float* dsp = seg_dsum + b * g.D + d;          // [s][b][d]
  for (int s0 = 0; s0 < g.S; s0 += kCarryBatch) {
    float st[kCarryBatch], ds[kCarryBatch];
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i) {
      const bool live = s0 + i < g.S - 1;            // segment S-1 has no end state
      st[i] = live ? slot[(int64_t)(s0 + i) * sstride] : 0.0f;
      ds[i] = live ? dsp[(int64_t)(s0 + i) * dstride] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i) {
      if (s0 + i < g.S) slot[(int64_t)(s0 + i) * sstride] = h;
      h = __builtin_fmaf(fast_exp2(a2 * ds[i]), h, st[i]);
    }
  }
}

static SelSeg make_seg(const SelArgs& a, const SelPlan& pl, int ns) {
  SelSeg g{};
  g.batch = a.batch;
  g.L = a.seqlen;
  g.D = a.dim;
  g.seg_len = pl.seg_len;
  g.N = ns;
  g.S = pl.segments;
  g.ngroups = (int)((a.dim + 63) / 64);
  g.gpb = std::min(2, g.ngroups);
  g.nblk = (g.ngroups + g.gpb - 1) / g.gpb;
  g.vec = selective_row_mode(a, pl) - 1;
  return g;
}


// B and C from channel-major (batch, dstate, seqlen) to the time-major rows the scan kernels
// read with scalar loads: one workgroup per (batch, 64 steps, tensor) through an LDS tile,
// reading 256-byte row pieces and writing one contiguous 64 * dstate block.
static __global__ __launch_bounds__(256) void bc_rows_kernel(const float* __restrict__ B, const float* __restrict__ C,
                                                      float* __restrict__ Bt, float* __restrict__ Ct, int64_t batch,
                                                      int64_t L, int N) {
  __shared__ float tile[64][65];
  const float* src = blockIdx.y == 0 ? B : C;
  float* dst = blockIdx.y == 0 ? Bt : Ct;
  const int64_t tiles = (L + 63) / 64;
  const int64_t b = (int64_t)blockIdx.x / tiles;
  const int64_t t0 = ((int64_t)blockIdx.x - b * tiles) * 64;
  const int cnt = (int)std::min<int64_t>(64, L - t0);
  for (int i = threadIdx.x; i < N * 64; i += 256) {
    const int n = i >> 6, tt = i & 63;
    if (tt < cnt) tile[n][tt] = src[(b * N + n) * L + t0 + tt];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < cnt * N; i += 256) {
    const int tt = i / N, n = i - tt * N;
    dst[(b * L + t0) * N + i] = tile[n][tt];
  }
}

// The segment state slots: the caller's buffer when one is given, else the workspace's.
static float* state_slots(const SelArgs& a, const SelPlan& pl) {
  return a.states != nullptr ? a.states : reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + pl.ws_state);
}

// Pass 1 and the carry: the state slots end up holding the state entering every segment
// (S > 1; nothing to do for a single segment).
template <int NS, bool BF16, int FL>
static hipError_t run_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  if (pl.segments <= 1) return hipSuccess;
  const SelSeg g = make_seg(a, pl, NS);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* st = state_slots(a, pl);
  float* ds = reinterpret_cast<float*>(ws + pl.ws_dsum);
  const int64_t per_seg = (int64_t)g.nblk * g.batch;
  const size_t lds1 = g.vec == 2 ? (size_t)g.gpb * 2 * 64 * kTileBytes  // x, delta tiles
                                  : lds_rows(NS, FL) ? (size_t)g.gpb * row_tile_lds(1) : 0;  // B row tiles
  hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 1, false, FL>), dim3((unsigned)(per_seg * (pl.segments - 1))),
                     dim3(64u * (unsigned)g.gpb), lds1, stream, a.x, a.delta, a.A, a.B, a.C, a.Dsk, a.z, a.h0,
                     (const float*)nullptr, a.y, a.h_last, st, ds, a.delta_bias, (const float*)nullptr,
                     (float*)nullptr, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nthr = g.batch * (int64_t)NS * g.D;
  hipLaunchKernelGGL(sel_carry_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream, a.A, a.h0, st,
                     (const float*)ds, g);
  return hipGetLastError();
}

template <int NS, bool BF16, int FL>
static hipError_t run_selective(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  hipError_t e = run_states<NS, BF16, FL>(a, pl, stream);
  if (e != hipSuccess) return e;
  const SelSeg g = make_seg(a, pl, NS);
  const float* st = pl.segments > 1 ? state_slots(a, pl) : nullptr;
  const int64_t per_seg = (int64_t)g.nblk * g.batch;
  const dim3 grid((unsigned)(per_seg * pl.segments)), block(64u * (unsigned)g.gpb);
  const size_t lds2 = g.vec == 2 ? (size_t)g.gpb * (a.z != nullptr ? 3 : 2) * 64 * kTileBytes
                                  : lds_rows(NS, FL) ? (size_t)g.gpb * row_tile_lds(2) : 0;  // B, C row tiles
  if (a.z != nullptr)
    hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 2, true, FL>), grid, block, lds2, stream, a.x, a.delta, a.A, a.B, a.C,
                       a.Dsk, a.z, a.h0, st, a.y, a.h_last, (float*)nullptr, (float*)nullptr, a.delta_bias,
                       (const float*)nullptr, (float*)nullptr, g);
  else
    hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 2, false, FL>), grid, block, lds2, stream, a.x, a.delta, a.A, a.B,
                       a.C, a.Dsk, a.z, a.h0, st, a.y, a.h_last, (float*)nullptr, (float*)nullptr, a.delta_bias,
                       (const float*)nullptr, (float*)nullptr, g);
  return hipGetLastError();
}

// Segment entering states of the plain form (no options), for the backward pass.
template <int NS, bool BF16>
hipError_t run_segment_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  return run_states<NS, BF16, 0>(a, pl, stream);
}

// Checkpoints for the backward pass: the state before every 2^kshift-th step of every
// segment, into ckpt[s][b][grp][j][row][lane] (NS + 1 rows per checkpoint).  With adj_mu
// (S > 1) the same pass folds each segment's adjoint from a zero adjoint at its end into
// adj_mu[s][b][n][d] (dy and the z gate give the read-out's gradient) and writes every
// segment's delta sum into the forward workspace's sums.  Without `local` the state slots
// already hold the segments' entering states (run_segment_states, or states the forward
// call kept) and the checkpoints are the states themselves; with `local` every segment
// starts from zero, the checkpoints carry their delta sums, and the carry then turns the
// end states this pass leaves in the slots into the entering states (the backward kernel
// adds their decayed contribution to each checkpoint).
// FX: the delta front end's bits (kFront, kSoftplus), so that the checkpoints, the delta sums
// and the decays of the adjoint fold use the step sizes the forward call used.
template <int NS, bool BF16, int FX>
static hipError_t run_ckpt_fl(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub, const float* dy,
                              float* adj_mu, bool local, hipStream_t stream) {
  SelSeg g = make_seg(a, pl, NS);
  g.kshift = kshift;
  g.nsub = nsub;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* st = pl.segments > 1 ? state_slots(a, pl) : nullptr;
  const int64_t per_seg = (int64_t)g.nblk * g.batch;
  const dim3 grid((unsigned)(per_seg * pl.segments)), block(64u * (unsigned)g.gpb);
  if (adj_mu != nullptr && pl.segments > 1) {
    float* ds = reinterpret_cast<float*>(ws + pl.ws_dsum);
    g.local = local ? 1 : 0;
    const float* carry = local ? nullptr : st;  // entering states (read), or
    float* ends = local ? st : nullptr;         // end states from zero (written)
    const size_t lds3 = lds_rows(NS, kAdj) ? (size_t)g.gpb * row_tile_lds(3, true) : 0;  // B, C row tiles
    if (a.z != nullptr)
      hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 3, true, kAdj | FX>), grid, block, lds3, stream, a.x, a.delta, a.A, a.B,
                         a.C, a.Dsk, a.z, a.h0, carry, (float*)nullptr, ends, ckpt, ds,
                         a.delta_bias, dy, adj_mu, g);
    else
      hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 3, false, kAdj | FX>), grid, block, lds3, stream, a.x, a.delta, a.A,
                         a.B, a.C, a.Dsk, a.z, a.h0, carry, (float*)nullptr, ends, ckpt, ds,
                         a.delta_bias, dy, adj_mu, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !local) return e;
    const int64_t nthr = g.batch * (int64_t)NS * g.D;
    hipLaunchKernelGGL(sel_carry_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream, a.A, a.h0, st,
                       (const float*)ds, g);
    return hipGetLastError();
  }
  const size_t lds3 = lds_rows(NS, 0) ? (size_t)g.gpb * row_tile_lds(3) : 0;  // B row tiles
  hipLaunchKernelGGL((sel_seq_kernel<NS, BF16, 3, false, FX>), grid, block, lds3, stream, a.x, a.delta, a.A, a.B, a.C,
                     a.Dsk, a.z, a.h0, st, (float*)nullptr, (float*)nullptr, ckpt, (float*)nullptr,
                     a.delta_bias, (const float*)nullptr, (float*)nullptr, g);
  return hipGetLastError();
}

template <int NS, bool BF16>
hipError_t run_checkpoints(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub, const float* dy,
                           float* adj_mu, bool local, hipStream_t stream) {
  if (a.softplus) return run_ckpt_fl<NS, BF16, kFront | kSoftplus>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
  if (a.delta_bias != nullptr) return run_ckpt_fl<NS, BF16, kFront>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
  return run_ckpt_fl<NS, BF16, 0>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
}

// Front end / hold variants: plain, exact hold, delta + bias (+ softplus), and both; each in
// the time-major and the channel-major layout.
template <int NS, bool BF16, int LAY>
static hipError_t run_options(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  const bool front = a.delta_bias != nullptr || a.softplus;
  const int fl = (a.exact_zoh ? kZoh : 0) | (front ? kFront : 0) | (a.softplus ? kSoftplus : 0);
  switch (fl) {
    case 0: return run_selective<NS, BF16, LAY>(a, pl, stream);
    case kZoh: return run_selective<NS, BF16, LAY | kZoh>(a, pl, stream);
    case kFront: return run_selective<NS, BF16, LAY | kFront>(a, pl, stream);
    case kFront | kSoftplus: return run_selective<NS, BF16, LAY | kFront | kSoftplus>(a, pl, stream);
    case kZoh | kFront: return run_selective<NS, BF16, LAY | kZoh | kFront>(a, pl, stream);
    case kZoh | kFront | kSoftplus: return run_selective<NS, BF16, LAY | kZoh | kFront | kSoftplus>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int NS, bool BF16>
hipError_t run_flags(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  if (!a.bdl) return run_options<NS, BF16, 0>(a, pl, stream);
  // channel-major B/C become time-major rows in the workspace first
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* bt = reinterpret_cast<float*>(ws + pl.ws_bc);
  float* ct = bt + a.batch * a.seqlen * NS;
  const int64_t tiles = (a.seqlen + 63) / 64;
  hipLaunchKernelGGL(bc_rows_kernel, dim3((unsigned)(a.batch * tiles), 2), dim3(256), 0, stream, a.B, a.C, bt, ct,
                     a.batch, a.seqlen, NS);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelArgs r = a;
  r.B = bt;
  r.C = ct;
  return run_options<NS, BF16, kBdl>(r, pl, stream);
}

// Explicit instances: the file is compiled once per state count (SSS_INST_NS = N) and once
// for the host part (plan and dispatch), so that the builds of the instances run in parallel.
#ifdef SSS_INST_NS
template hipError_t run_flags<SSS_INST_NS, false>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_flags<SSS_INST_NS, true>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_segment_states<SSS_INST_NS, false>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_segment_states<SSS_INST_NS, true>(const SelArgs&, const SelPlan&, hipStream_t);
template hipError_t run_checkpoints<SSS_INST_NS, false>(const SelArgs&, const SelPlan&, float*, int, int, const float*,
                                                        float*, bool, hipStream_t);
template hipError_t run_checkpoints<SSS_INST_NS, true>(const SelArgs&, const SelPlan&, float*, int, int, const float*,
                                                       float*, bool, hipStream_t);
#else
int selective_row_mode(const SelArgs& a, const SelPlan& pl) {
  if (!a.bdl) return 0;
  const int64_t piece = a.bf16 ? 8 : 4;  // steps per 16-byte piece of a channel-major row
  const int64_t tile = kTileBytes / (a.bf16 ? 2 : 4);
  if (a.dstate <= 16 && a.seqlen % tile == 0 && pl.seg_len % tile == 0) return 3;
  return (a.seqlen % piece == 0 && pl.seg_len % piece == 0) ? 2 : 1;
}
#define SSS_EXTERN_INSTANCES(N)                                                                        \
  extern template hipError_t run_flags<N, false>(const SelArgs&, const SelPlan&, hipStream_t);           \
  extern template hipError_t run_flags<N, true>(const SelArgs&, const SelPlan&, hipStream_t);            \
  extern template hipError_t run_segment_states<N, false>(const SelArgs&, const SelPlan&, hipStream_t);  \
  extern template hipError_t run_segment_states<N, true>(const SelArgs&, const SelPlan&, hipStream_t);            \
  extern template hipError_t run_checkpoints<N, false>(const SelArgs&, const SelPlan&, float*, int, int, const float*, \
                                                      float*, bool, hipStream_t);                                   \
  extern template hipError_t run_checkpoints<N, true>(const SelArgs&, const SelPlan&, float*, int, int, const float*,  \
                                                     float*, bool, hipStream_t);
SSS_EXTERN_INSTANCES(1)
SSS_EXTERN_INSTANCES(2)
SSS_EXTERN_INSTANCES(4)
SSS_EXTERN_INSTANCES(8)
SSS_EXTERN_INSTANCES(16)
SSS_EXTERN_INSTANCES(32)
SSS_EXTERN_INSTANCES(64)
#undef SSS_EXTERN_INSTANCES

// ------------------------------------------------------------------ host side
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

SelPlan plan_selective(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus, bool bdl,
                       size_t max_ws) {
  SelPlan pl{};
  // segments start on whole load batches: 2 steps, or whole channel-major tiles (32 steps)
  const int64_t unit = bdl ? 32 : kStepsPerBatch;
  const int64_t groups = batch * ((dim + 63) / 64);
  const int64_t simds = (int64_t)std::max(num_cus, 1) * 4;
  // One wave per (channel group, segment).  Splitting time costs a second pass over the
  // inputs, so it is only worth it when the channel groups alone leave most SIMDs idle;
  // then aim at ~20 waves per SIMD: short segments keep every SIMD busy to the end.  Below
  // 64 steps a segment's fixed costs (entering state, end state, carry) outweigh that
  // (measured: 8 x 2048 x 1536 at 32 segments 0.166 ms, at 64 0.175; 16 x 2048 x 1024 at 32
  // segments 0.184, at 64 0.198; 2 x 8192 x 2560 at 128 segments 0.229, at 256 0.253).
  int64_t S = 1;
  if (groups < 2 * simds) {
    const int64_t target = simds * env_int("SSS_WAVES_PER_SIMD", 20);
    S = std::max<int64_t>(1, (target + groups / 2) / groups);
    // segments of >= 64 steps, or >= 32 where even those would leave most SIMDs without a
    // wave: such small calls are bound by each wave's serial walk (2 x 512 x 64: 41 us at 8
    // segments, 28 us at 16)
    const int64_t min_len = groups * std::max<int64_t>(1, seqlen / 64) >= simds ? 64 : 32;
    S = std::min<int64_t>(S, std::max<int64_t>(1, seqlen / min_len));
    S = std::min<int64_t>(S, 4096);
  }
  const int forced = env_int("SSS_FORCE_SEGMENTS", 0);
  if (forced > 0) S = std::min<int64_t>(forced, (seqlen + unit - 1) / unit);
  if (S < 1) S = 1;
  if (max_ws > 0 && S > 1) {
    // workspace of S segments <= S * (states + delta sums) + two 256-byte roundings (+ B/C rows)
    const int64_t per_seg = batch * dim * (dstate + 1) * 4;
    const int64_t fixed = 512 + (bdl ? (int64_t)align_up((size_t)2 * batch * seqlen * dstate * 4, 256) : 0);
    const int64_t room = (int64_t)max_ws - fixed;
    S = std::max<int64_t>(1, std::min<int64_t>(S, room > 0 ? room / per_seg : 1));
  }
  // buffer offsets inside one segment (seg_len rows of dim fp32 values) must stay below
  // 2^30 bytes; dim <= 2^24 is checked by the caller, so max_len >= 16 steps (the B/C row
  // pointers advance by dstate floats per step, also kept below 2^30 bytes)
  const int64_t row_bytes = std::max(dim, dstate) * 4;
  const int64_t max_len = std::max<int64_t>(unit, ((int64_t)1 << 30) / row_bytes / unit * unit);
  int64_t seg_len = (seqlen + S - 1) / S;
  seg_len = (seg_len + unit - 1) / unit * unit;
  seg_len = std::min(seg_len, max_len);
  S = (seqlen + seg_len - 1) / seg_len;
  pl.segments = (int)S;
  pl.seg_len = seg_len;
  // workspace: segment states / entering states [S][batch][dstate][dim], segment sums of
  // delta [S][batch][dim]; channel-major calls add time-major copies of B and C
  const size_t st_bytes = S > 1 ? align_up((size_t)S * batch * dstate * dim * 4, 256) : 0;
  const size_t ds_bytes = S > 1 ? align_up((size_t)S * batch * dim * 4, 256) : 0;
  const size_t bc_bytes = bdl ? align_up((size_t)2 * batch * seqlen * dstate * 4, 256) : 0;
  pl.ws_state = 0;
  pl.ws_dsum = st_bytes;
  pl.ws_bc = st_bytes + ds_bytes;
  pl.ws_total = st_bytes + ds_bytes + bc_bytes;
  return pl;
}

template <bool BF16>
static hipError_t dispatch_n(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_flags<1, BF16>(a, pl, stream);
    case 2: return run_flags<2, BF16>(a, pl, stream);
    case 4: return run_flags<4, BF16>(a, pl, stream);
    case 8: return run_flags<8, BF16>(a, pl, stream);
    case 16: return run_flags<16, BF16>(a, pl, stream);
    case 32: return run_flags<32, BF16>(a, pl, stream);
    case 64: return run_flags<64, BF16>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_selective(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  return a.bf16 ? dispatch_n<true>(a, pl, stream) : dispatch_n<false>(a, pl, stream);
}

template <bool BF16>
static hipError_t dispatch_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_segment_states<1, BF16>(a, pl, stream);
    case 2: return run_segment_states<2, BF16>(a, pl, stream);
    case 4: return run_segment_states<4, BF16>(a, pl, stream);
    case 8: return run_segment_states<8, BF16>(a, pl, stream);
    case 16: return run_segment_states<16, BF16>(a, pl, stream);
    case 32: return run_segment_states<32, BF16>(a, pl, stream);
    case 64: return run_segment_states<64, BF16>(a, pl, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_segment_states(const SelArgs& a, const SelPlan& pl, hipStream_t stream) {
  return a.bf16 ? dispatch_states<true>(a, pl, stream) : dispatch_states<false>(a, pl, stream);
}

template <bool BF16>
static hipError_t dispatch_ckpt(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub,
                                const float* dy, float* adj_mu, bool local, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return run_checkpoints<1, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    case 2: return run_checkpoints<2, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    case 4: return run_checkpoints<4, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    case 8: return run_checkpoints<8, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    case 16: return run_checkpoints<16, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    case 32: return run_checkpoints<32, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    case 64: return run_checkpoints<64, BF16>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_checkpoints(const SelArgs& a, const SelPlan& pl, float* ckpt, int kshift, int nsub, const float* dy,
                              float* adj_mu, bool local, hipStream_t stream) {
  return a.bf16 ? dispatch_ckpt<true>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream)
                : dispatch_ckpt<false>(a, pl, ckpt, kshift, nsub, dy, adj_mu, local, stream);
}

#endif  // SSS_INST_NS

}  // namespace sss
