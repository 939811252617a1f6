// selective_bwd.hip -- gfx950 kernels for the gradients of the selective scan.
//
// Training needs the gradients of the scan's inputs.  "Selective Scan trong Mamba toi uu
// chuoi dai the nao?" (section "Recomputation: doi mot it compute lay it memory hon"):
// the states are not kept from the forward pass but recomputed.  With
//   a_t = exp(delta_t A_n), h_t = a_t h_{t-1} + delta_t B_t[n] x_t,
//   y_t = (sum_n C_t[n] h_t[n] + D x_t) silu(z_t),
// the adjoint lambda_t = dL/dh_t runs backwards in time with the same affine structure,
//   lambda_t = C_t dv_t + a_{t+1} lambda_{t+1},   dv_t = dy_t silu(z_t),
// and every gradient is a per-step product of lambda_t with forward quantities:
//   dx_t = D dv_t + sum_n lambda_t delta_t B_t,  ddelta_t = sum_n lambda_t (B_t x_t + A a_t h_{t-1}),
//   dA_n = sum lambda_t delta_t a_t h_{t-1},     dB_t[n] = sum_d lambda_t delta_t x_t,
//   dC_t[n] = sum_d dv_t h_t,  dD = sum dv_t x_t,  dz_t = dy_t v_t silu'(z_t),  dh0 = a_0 lambda_0.
//
// Mapping (lanes = 64 adjacent channels, time split into the forward pass's segments):
//   1.+2. the forward scan's checkpoint pass (selective_scan.hip) runs every segment from a
//      zero state: it stores that state and the delta sum before every K-th step, the
//      segment's end state, and, from the decays it forms anyway, each segment's adjoint
//      folded from zero at its end (mu = a (mu + C dv) backwards, summed forwards as
//      sum_t a_first..a_t C_t dv_t); the forward carry turns the end states into the state
//      entering every segment.  Since the scan is linear in its state, the true state at a
//      checkpoint is the stored one plus exp2(A' * S) times the entering state (S the delta
//      sum before it), which the main kernel adds once per checkpoint.  (When the forward
//      call kept the entering states, the checkpoint pass starts from them instead.)
//   3. sel_bwd_carry: the adjoint entering every segment from its right end (from dh_last);
//   4. sel_bwd_kernel takes each segment's K-step sub-chunks in reverse order: their states
//      are re-formed in registers from the checkpoint and the adjoint walks them backwards, writing dx,
//      ddelta, dz and per-wave partial sums of dB/dC (a cross-lane reduce-scatter over the
//      64 channels) and per-segment partials of dA/dD;
//   5. small kernels add the partials up.
#include "common.h"
#include "front.h"
#include "kernels.h"

#include <algorithm>

namespace sss {

struct BwdSeg {
  int64_t batch, L, D, seg_len;
  int S, ngroups, nsub, K;
  int local;  // checkpoints from zero-started segments: add the decayed entering state
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bwd_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

template <bool BF16>
__device__ __forceinline__ float ld_io(__amdgpu_buffer_rsrc_t r, int vo, int so) {
  if (BF16) return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0) << 16);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
}

typedef __attribute__((address_space(3))) void lds_void;

// one element per lane copied straight into LDS (the lane's dword of the destination; a
// 2-byte element lands zero-extended in its low half).  The size operand must be a literal.
template <bool BF16>
__device__ __forceinline__ void copy_io_lds(__amdgpu_buffer_rsrc_t r, lds_void* dst, int vo, int so) {
  if constexpr (BF16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 2, vo, so, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, vo, so, 0, 0);
}

// NS rows of 64 dwords (a checkpoint as stored) copied straight into LDS at dst: 1 KB (four
// rows) per copy, lane i taking bytes 16 i .. 16 i + 15 of it, or a row per copy below 4 rows
template <int NS>
__device__ __forceinline__ void copy_rows_lds(__amdgpu_buffer_rsrc_t r, uint32_t* dst, int lane) {
  if constexpr (NS % 4 == 0) {
#pragma unroll
    for (int c = 0; c < NS / 4; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + c * 256), 16, lane * 16, c * 1024, 0, 0);
  } else {
#pragma unroll
    for (int n = 0; n < NS; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + n * 64), 4, lane * 4, n * 256, 0, 0);
  }
}

__device__ __forceinline__ float ld_f32(__amdgpu_buffer_rsrc_t r, int vo, int so) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
}

__device__ __forceinline__ void st_f32(float v, __amdgpu_buffer_rsrc_t r, int vo, int so) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, vo, so, 2);
}

// a h_t = h_{t+1} - (delta x)_t B_t, the input term rounded exactly as the forward step
// rounded it (not fused), so that a zero a h_t comes back as zero
__device__ __forceinline__ float minus_input(float h_next, float dx, float b) {
#pragma clang fp contract(off)
  const float p = dx * b;
  return h_next - p;
}

// silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
__device__ __forceinline__ float sigmoid_f(float z) { return fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// checkpoint spacing K: the K+1 states of a sub-chunk live in registers next to the adjoint
// (measured on the 1 x 65536 x 5120 N=16 layer: K=2 11.7 ms; K=4 spills or, with a 512-VGPR
// budget, runs one wave per SIMD: 17 ms)
constexpr int bwd_k(int ns) { return ns >= 64 ? 1 : ns >= 16 ? 2 : ns >= 8 ? 4 : 8; }
// sub-chunks per checkpoint: at 16 states a checkpoint every 2K steps, the odd sub-chunks
// advancing it by K steps first (half the checkpoint bytes written and read, for K more
// forward steps per 2K)
constexpr int bwd_r(int ns) { return ns == 16 ? 2 : 1; }
// resident waves per SIMD of the main kernel: three at 16 states (168 VGPRs; 2 waves ran it
// at 5.1-5.2 ms on that layer, 3 at 4.6 ms)
constexpr int bwd_min_waves(int ns) { return ns >= 32 ? 1 : ns >= 16 ? 3 : 2; }

// Common prologue: (wave, batch, segment) of this workgroup and the lane's channel.
struct BwdLane {
  int lane, grp, s;
  int64_t b, d0, dc, tbeg;
  int loff, len;
  bool real;  // false for lanes mirroring channel D-1 past the end
};

__device__ __forceinline__ BwdLane bwd_lane(const BwdSeg& g, int seg_offset) {
  BwdLane r;
  r.lane = threadIdx.x & 63;
  uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
  r.grp = (int)(lid % (uint32_t)g.ngroups);
  lid /= (uint32_t)g.ngroups;
  r.b = (int64_t)(lid % (uint32_t)g.batch);
  r.s = (int)(lid / (uint32_t)g.batch) + seg_offset;
  r.d0 = (int64_t)r.grp * 64;
  r.real = r.d0 + r.lane < g.D;
  r.dc = min(r.d0 + r.lane, g.D - 1);
  r.loff = (int)(r.dc - r.d0);
  r.tbeg = (int64_t)r.s * g.seg_len;
  r.len = (int)(min(r.tbeg + g.seg_len, g.L) - r.tbeg);
  return r;
}

// ------------------------------------------------------------------ 3. reverse carry
// One thread per (b, n, d), in place: slot[s] := adjoint entering segment s from its right
// end (dh_last for the last segment), then mu_{s-1} = exp2(A' sum delta_s) mu_s + mu_loc[s].
__global__ __launch_bounds__(256) void sel_bwd_carry(const float* __restrict__ A, const float* __restrict__ dh_last,
                                                     float* slots, const float* __restrict__ seg_dsum, int64_t batch,
                                                     int64_t D, int N, int S) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_b = (int64_t)N * D;
  if (idx >= batch * per_b) return;
  const int64_t b = idx / per_b, rem = idx - b * per_b;
  const int64_t n = rem / D, d = rem - n * D;
  const float a2 = fmaxf(A[d * N + n] * kLog2e, -kFltMax);
  float cur = dh_last ? dh_last[(b * D + d) * N + n] : 0.0f;
  const int64_t sstride = batch * per_b, dstride = batch * D;
  float* slot = slots + b * per_b + rem;
  const float* dsp = seg_dsum + b * D + d;
  for (int s1 = S - 1; s1 >= 0; s1 -= 8) {
    float lo[8], ds[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s1 - i;
      const bool live = s >= 1;  // segment 0 has no local fold
      lo[i] = live ? slot[(int64_t)s * sstride] : 0.0f;
      ds[i] = live ? dsp[(int64_t)s * dstride] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = s1 - i;
      if (s >= 0) slot[(int64_t)s * sstride] = cur;
      cur = __builtin_fmaf(fast_exp2(a2 * ds[i]), cur, lo[i]);
    }
  }
}

// ------------------------------------------------------------------ cross-lane reduce-scatter
// V values per lane -> after the levels 32, 16, 8, 4, 2, 1 (lane bit of the level) each lane
// holds V >> min(6, log2 V) values, each summed over all 64 lanes; value index =
// (lane >> (6 - levels)) * keep + i.  Level LV halves the CNT live values: lanes with the
// level's bit set keep the upper half, the others the lower half, and each adds its partner's
// copy of the half it keeps; once one value is left the levels just add the partner's value.
// Partners: v_permlane32_swap / v_permlane16_swap exchange the halves of two registers across
// 32 / 16 lanes in one instruction (lane bits 5 and 4); within a row of 16 lanes DPP
// row_mirror, row_half_mirror and the quad permutations pair lanes that differ in bit 3, 2,
// 1 and 0 and agree on every higher bit -- the same pairs of value sets as an xor exchange.
__device__ __forceinline__ uint32_t bwd_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bwd_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// v + (v of the partner lane) for every lane, the partner given by the DPP control of
// level LV (2: row_mirror, 3: row_half_mirror, 4: quad_perm [2,3,0,1], 5: quad_perm
// [1,0,3,2]): one v_add_f32_dpp.  (The s_nop covers the DPP read-after-VALU-write hazard.)
template <int LV>
__device__ __forceinline__ float dpp_self_sum(float v) {
  float r;
  if constexpr (LV == 2)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  else if constexpr (LV == 3)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  else if constexpr (LV == 4)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  else
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  return r;
}

// Levels 2 and 3 pair lanes across 4-lane banks (bit 3: banks 0,1 against 2,3; bit 2: banks
// 0,2 against 1,3), so each half of the lanes takes its kept value in one DPP add whose bank
// mask writes only that half: low lanes a + partner's a, high lanes b + partner's b.  (The
// result register is written in two halves; it must not be a or b, whose low lanes the
// second add still reads from the partners.)
template <int LV>
__device__ __forceinline__ float dpp_split_sum(float a, float b) {
  float r;
  if constexpr (LV == 2)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_mirror row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %0, %2, %2 row_mirror row_mask:0xf bank_mask:0xc"
        : "=&v"(r) : "v"(a), "v"(b));
  else
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa"
        : "=&v"(r) : "v"(a), "v"(b));
  return r;
}

// a: the value lanes without the level's bit keep, b: the value lanes with it keep
template <int LV>
__device__ __forceinline__ float pair_sum(float a, float b, bool hi) {
  if constexpr (LV == 0 || LV == 1) {
    // the upper lanes of the first register trade places with the lower lanes of the second:
    // afterwards every lane holds its own kept value and its partner's copy of it
    const auto r = LV == 0 ? __builtin_amdgcn_permlane32_swap(bwd_u32(a), bwd_u32(b), false, false)
                           : __builtin_amdgcn_permlane16_swap(bwd_u32(a), bwd_u32(b), false, false);
    const uint32_t r0 = r[0], r1 = r[1];  // elements copied out before the casts
    return bwd_f32(r0) + bwd_f32(r1);
  } else {
    constexpr int ctrl = LV == 2 ? 0x140 : LV == 3 ? 0x141 : LV == 4 ? 0x4E : 0xB1;
    const float keep = hi ? b : a;
    const float send = hi ? a : b;
    return keep + bwd_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)bwd_u32(send), ctrl, 0xF, 0xF, false));
  }
}

template <int LV, int CNT, int V>
__device__ __forceinline__ void reduce_scatter_level(float (&p)[V], int lane) {
  if constexpr (LV < 6) {
    const bool hi = (lane & (32 >> LV)) != 0;
    if constexpr (CNT > 1) {
      constexpr int half = CNT / 2;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        if constexpr (LV == 2 || LV == 3) p[i] = dpp_split_sum<LV>(p[i], p[half + i]);
        else p[i] = pair_sum<LV>(p[i], p[half + i], hi);
      }
      reduce_scatter_level<LV + 1, half, V>(p, lane);
    } else {
      if constexpr (LV >= 2) p[0] = dpp_self_sum<LV>(p[0]);
      else p[0] = pair_sum<LV>(p[0], p[0], hi);
      reduce_scatter_level<LV + 1, 1, V>(p, lane);
    }
  }
}

template <int V>
__device__ __forceinline__ void reduce_scatter(float (&p)[V], int lane) {
  reduce_scatter_level<0, V, V>(p, lane);
}

constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v / 2); }

// ------------------------------------------------------------------ 4. main backward pass
// Checkpoints (the state before every K-th step, from the forward scan's PASS 3) are taken
// in reverse order; for each K-step sub-chunk the states are re-formed in registers and the
// adjoint walks the sub-chunk backwards.  A checkpoint and the inputs of the steps it
// covers reach LDS through direct-to-LDS buffer loads one checkpoint group ahead, so no
// VGPRs wait on them (a prefetch into a second register slot spilled at 168 VGPRs).
// scheduling barrier between the phases of a recomputed step: memory, scalar and LDS
// instructions may cross it, VALU instructions may not
constexpr int kBwdPhase = 0x3FC;

// FX: the delta front end's bits (kFront: the step size is delta + bias[d]; kSoftplus:
// softplus of that).  The step sizes are formed from the staged raw delta exactly as the
// forward call formed them; ddelta is then the gradient with respect to the raw delta (the
// step size's gradient times sigmoid(delta + bias) under softplus, formed from the step size
// at the store).  The bias gradient is summed from ddelta by a pass of its own: a running sum
// here would hold one more VGPR through the loop, which at 16 states spills.
template <int NS, bool BF16, bool HAS_Z, int FX>
__global__ __launch_bounds__(64, bwd_min_waves(NS)) void sel_bwd_kernel(
    const void* __restrict__ x, const void* __restrict__ delta, const float* __restrict__ A,
    const float* __restrict__ Bm, const float* __restrict__ Cm, const float* __restrict__ Dsk,
    const void* __restrict__ z, const float* __restrict__ dy, const float* __restrict__ dh_last,
    const float* __restrict__ mu_right, const float* __restrict__ ckpt, const float* __restrict__ hin,
    float* __restrict__ dx,
    float* __restrict__ ddelta, float* __restrict__ dz, float* __restrict__ part_bc, float* __restrict__ part_a,
    float* __restrict__ part_d, float* __restrict__ dh0, const float* __restrict__ dbias, BwdSeg g) {
  constexpr int K = bwd_k(NS);
  constexpr int R = bwd_r(NS);
  constexpr int ES = BF16 ? 2 : 4;
  // dB and dC partials of one step go through one reduce-scatter of 2 NS values; from 16
  // states on through two of NS (fewer live registers)
  constexpr bool kMerged = NS < 16;
  constexpr int NV = kMerged ? 2 * NS : NS;            // values per reduce-scatter
  constexpr int LV = ilog2c(NV) < 6 ? ilog2c(NV) : 6;  // its levels
  constexpr int KEEP = NV >> LV;
  const BwdLane q = bwd_lane(g, 0);
  const int64_t chl = (q.b * g.D + q.dc) * NS;  // (b, d) row of dh_last / dh0

  float a2[NS], mu[NS], dacc[NS];  // A' = A log2 e (for exp2; A itself is A' ln 2), clamped
  // the adjoint entering from the right: the carried one (state n at stride D), else dh_last
  // (contiguous), else zero -- one source for all n, so that the loads go out together
  const float* mu_src = g.S > 1 ? mu_right + ((int64_t)q.s * g.batch + q.b) * NS * g.D + q.dc
                                : (dh_last ? dh_last + chl : nullptr);
  const int64_t mu_stride = g.S > 1 ? g.D : 1;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    a2[n] = fmaxf(A[q.dc * NS + n] * kLog2e, -kFltMax);
    mu[n] = 0.0f;
    dacc[n] = 0.0f;
  }
  if (mu_src != nullptr) {
#pragma unroll
    for (int n = 0; n < NS; ++n) mu[n] = mu_src[n * mu_stride];
  }
  const float Dd = Dsk ? Dsk[q.dc] : 0.0f;
  float ddacc = 0.0f;

  const int64_t row0 = (q.b * g.L + q.tbeg) * g.D + q.d0;
  const __amdgpu_buffer_rsrc_t rx = bwd_rsrc((const char*)x + row0 * ES);
  const __amdgpu_buffer_rsrc_t rd = bwd_rsrc((const char*)delta + row0 * ES);
  const __amdgpu_buffer_rsrc_t rz = bwd_rsrc(HAS_Z ? (const char*)z + row0 * ES : (const char*)x);
  const __amdgpu_buffer_rsrc_t rg = bwd_rsrc(dy + row0);
  const __amdgpu_buffer_rsrc_t rdx = bwd_rsrc(dx + row0);
  const __amdgpu_buffer_rsrc_t rdd = bwd_rsrc(ddelta + row0);
  const __amdgpu_buffer_rsrc_t rdz = bwd_rsrc(HAS_Z ? dz + row0 : dx + row0);
  // checkpoint j of this wave: [s][b][grp][j][row][lane], one contiguous 256-byte row per
  // state and one for the delta sum before it (written for zero-started segments)
  auto ck_rsrc = [&](int j) {
    return bwd_rsrc(ckpt + ((((int64_t)q.s * g.batch + q.b) * g.ngroups + q.grp) * g.nsub + j) * (NS + 1) * 64);
  };
  const int rs = (int)(g.D * ES), rs4 = (int)(g.D * 4);
  const int vo = q.loff * ES, vo4 = q.loff * 4;
  const float* Br = Bm + (q.b * g.L + q.tbeg) * NS;
  const float* Cr = Cm + (q.b * g.L + q.tbeg) * NS;
  const int last = (q.len - 1) / K;

  // LDS staging (one wave per workgroup).  A checkpoint group is the R sub-chunks (KC = R K
  // steps) that start from one checkpoint.  Its checkpoint (NS rows of 256 B, as stored) and,
  // per step, one dword per lane of x, delta, dy and z are copied into LDS by buffer loads
  // that write LDS directly (no VGPRs held), issued one group ahead: the group's last
  // sub-chunk issues the next group's copies once it has read its own inputs.  A 2-byte
  // element lands zero-extended in the low half of the lane's dword.  Every copy reads the
  // same in-range addresses the lanes' own loads would (rows clamped to the segment, lanes
  // past the last channel on channel D-1).
  constexpr int KC = K * R;
  constexpr int kOffX = (NS + 1) * 64, kOffD = kOffX + KC * 64, kOffG = kOffD + KC * 64, kOffZ = kOffG + KC * 64;
  // with the delta front end each group's step sizes replace its raw deltas in place once the
  // group has landed
  __shared__ __attribute__((aligned(16))) uint32_t stage[kOffZ + (HAS_Z ? KC * 64 : 0)];
  // the lane's bias, read at each group's conversion (kept out of the VGPR budget)
  __shared__ float dbias_s[(FX & kFront) != 0 ? 64 : 1];
  if constexpr ((FX & kFront) != 0) dbias_s[q.lane] = dbias != nullptr ? dbias[q.dc] : 0.0f;
  auto lds_at = [&](int word) { return (lds_void*)&stage[word]; };
  auto issue_group = [&](int grp_j) {
    const __amdgpu_buffer_rsrc_t rk = ck_rsrc(grp_j);
    copy_rows_lds<NS>(rk, stage, q.lane);
    if (g.local) __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_at(NS * 64), 4, q.lane * 4, NS * 256, 0, 0);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int t_ = min(grp_j * KC + i, q.len - 1);
      copy_io_lds<BF16>(rx, lds_at(kOffX + i * 64), vo, t_ * rs);
      copy_io_lds<BF16>(rd, lds_at(kOffD + i * 64), vo, t_ * rs);
      copy_io_lds<false>(rg, lds_at(kOffG + i * 64), vo4, t_ * rs4);
      if constexpr (HAS_Z) copy_io_lds<BF16>(rz, lds_at(kOffZ + i * 64), vo, t_ * rs);
    }
  };
  // a staged element of the lane: bf16 bits widened to fp32
  auto lds_in = [&](int word) {
    const uint32_t u = stage[word + q.lane];
    return __builtin_bit_cast(float, BF16 ? u << 16 : u);
  };
  auto lds_f32 = [&](int word) { return __builtin_bit_cast(float, stage[word + q.lane]); };
  // a staged delta: the raw one, or the step size the front end made of it
  auto lds_dl = [&](int word) { return (FX & kFront) != 0 ? lds_f32(word) : lds_in(word); };

  float xs[1][K], ds[1][K], gs[1][K], zs[1][K];
#define BWD_LOAD(SLOT, J)                                                                  \
  do {                                                                                     \
    const int li_ = ((J) % R) * K; /* the sub-chunk's first step within its group */       \
    _Pragma("unroll") for (int i = 0; i < K; ++i) {                                        \
      xs[SLOT][i] = lds_in(kOffX + (li_ + i) * 64);                                        \
      ds[SLOT][i] = lds_dl(kOffD + (li_ + i) * 64);                                        \
      gs[SLOT][i] = lds_f32(kOffG + (li_ + i) * 64);                                       \
      if (HAS_Z) zs[SLOT][i] = lds_in(kOffZ + (li_ + i) * 64);                             \
    }                                                                                      \
  } while (0)

#define BWD_CHUNK(SLOT, J)                                                                 \
  do {                                                                                     \
    const int tb = (J) * K;                                                                \
    const int k = min(K, q.len - tb);                                                      \
    float hs[K + 1][NS], ea[K][NS]; /* states and decays of the sub-chunk */               \
    _Pragma("unroll") for (int n = 0; n < NS; ++n) hs[0][n] = h0[n];                       \
    if (R == 2 && ((J) & 1)) { /* the checkpoint is K steps before the sub-chunk */        \
      _Pragma("unroll") for (int i = 0; i < K; ++i) {                                      \
        const int ta = ((J) - 1) * K + i;                                                  \
        const float dla = da[i];                                                           \
        const float dxa = dla * xa[i];                                                     \
        const float* Ba = Br + ta * NS;                                                    \
        /* phased like the steps below; the decays go through ea[0], not yet in use */     \
        float ba_[NS];                                                                     \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) ba_[n] = Ba[n];                     \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) ea[0][n] = dla * a2[n];             \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        __builtin_amdgcn_s_setprio(2);                                                     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) ea[0][n] = fast_exp2(ea[0][n]);     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        __builtin_amdgcn_s_setprio(0);                                                     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        _Pragma("unroll") for (int n = 0; n < NS; ++n)                                     \
          hs[0][n] = __builtin_fmaf(ea[0][n], hs[0][n], dxa * ba_[n]);                     \
      }                                                                                    \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < K; ++i) {                                        \
      if (i < k) {                                                                         \
        const float* Bt = Br + (tb + i) * NS;                                              \
        const float dxv = ds[SLOT][i] * xs[SLOT][i];                                       \
        /* arguments, then the exps at a raised wave priority, then the updates (as the    \
           forward step: the other waves' VALU work pairs more often); the B_t row is       \
           loaded ahead of the phases */                                                   \
        float bt_[NS];                                                                     \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) bt_[n] = Bt[n];                     \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) ea[i][n] = ds[SLOT][i] * a2[n];     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        __builtin_amdgcn_s_setprio(2);                                                     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) ea[i][n] = fast_exp2(ea[i][n]);     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        __builtin_amdgcn_s_setprio(0);                                                     \
        __builtin_amdgcn_sched_barrier(kBwdPhase);                                         \
        _Pragma("unroll") for (int n = 0; n < NS; ++n)                                     \
          hs[i + 1][n] = __builtin_fmaf(ea[i][n], hs[i][n], dxv * bt_[n]);                 \
      }                                                                                    \
    }                                                                                      \
    _Pragma("unroll") for (int i = K - 1; i >= 0; --i) {                                   \
      if (i < k) {                                                                         \
        const int t = tb + i;                                                              \
        const float xv = xs[SLOT][i], dl = ds[SLOT][i], gy = gs[SLOT][i];                  \
        const float* Bt = Br + t * NS;                                                     \
        const float* Ct = Cr + t * NS;                                                     \
        float dv = gy, zv = 0.0f, sg = 0.0f;                                               \
        if (HAS_Z) {                                                                       \
          zv = zs[SLOT][i];                                                                \
          sg = sigmoid_f(zv);                                                              \
          dv = gy * zv * sg;                                                               \
        }                                                                                  \
        /* pv: this step's dB (first NS) and dC (last NS) partials of the lane's channel;  \
           lanes mirroring channel D-1 contribute zero */                                   \
        const float dvm = q.real ? dv : 0.0f;                                              \
        const float dxm = q.real ? dl * xv : 0.0f;                                         \
        float vsum = Dd * xv;                                                              \
        float* rowp = part_bc + (((int64_t)q.grp * g.batch + q.b) * g.L + q.tbeg + t) * (2 * NS); \
        const bool writer = (q.lane & ((1 << (6 - LV)) - 1)) == 0;                         \
        const int widx = (q.lane >> (6 - LV)) * KEEP;                                      \
        float pv[kMerged ? 2 * NS : NS], pc[kMerged ? 1 : NS];                             \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) {                                   \
          vsum = __builtin_fmaf(Ct[n], hs[i + 1][n], vsum);                                \
          if constexpr (kMerged) pv[NS + n] = dvm * hs[i + 1][n];                          \
          else pc[n] = dvm * hs[i + 1][n];                                                 \
        }                                                                                  \
        if constexpr (!kMerged) {                                                          \
          reduce_scatter<NV>(pc, q.lane);                                                  \
          if (writer) {                                                                    \
            _Pragma("unroll") for (int e = 0; e < KEEP; ++e) rowp[NS + widx + e] = pc[e];  \
          }                                                                                \
        }                                                                                  \
        /* slb = sum_n lam_n B_t[n] (dx takes it times delta, ddelta times x); ga: the A   \
           term of ddelta over ln 2 */                                                     \
        float slb = 0.0f, ga = 0.0f;                                                       \
        const float dxi = dl * xv;                                                         \
        _Pragma("unroll") for (int n = 0; n < NS; ++n) {                                   \
          const float a = ea[i][n];                                                        \
          const float lam = __builtin_fmaf(Ct[n], dv, mu[n]);                              \
          slb = __builtin_fmaf(lam, Bt[n], slb);                                           \
          /* a h_t: the sub-chunk's first state is not kept, so the first step forms it    \
             from the state after the step; the others have h_t in registers */            \
          const float ah = i > 0 ? a * hs[i > 0 ? i : 1][n] : minus_input(hs[i + 1][n], dxi, Bt[n]); \
          const float lah = lam * ah;                                                      \
          ga = __builtin_fmaf(lah, a2[n], ga); /* ah = 0 keeps A = -inf finite */          \
          dacc[n] = __builtin_fmaf(lah, dl, dacc[n]);                                      \
          pv[n] = lam * dxm;                                                               \
          mu[n] = a * lam;                                                                 \
        }                                                                                  \
        const float gx = __builtin_fmaf(slb, dl, Dd * dv);                                 \
        const float gd = slb * xv;                                                         \
        ddacc = __builtin_fmaf(dv, xv, ddacc);                                             \
        st_f32(gx, rdx, vo4, t * rs4);                                                     \
        float gdd = __builtin_fmaf(ga, kLn2, gd);                                          \
        if constexpr ((FX & kSoftplus) != 0) gdd *= softplus_slope_of_step(dl);            \
        st_f32(gdd, rdd, vo4, t * rs4);                                                    \
        if (HAS_Z) st_f32(gy * vsum * sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f), rdz, vo4, t * rs4); \
        reduce_scatter<kMerged ? 2 * NS : NS>(pv, q.lane);                                 \
        if (writer) {                                                                      \
          _Pragma("unroll") for (int e = 0; e < KEEP; ++e) rowp[widx + e] = pv[e];         \
        }                                                                                  \
      }                                                                                    \
    }                                                                                      \
  } while (0)

  // Zero-started segments: the state entering the segment, [n][lane] in LDS, for the
  // checkpoints' correction (the state at a checkpoint is the one from zero plus
  // exp2(A' * S) times the entering state, S the delta sum of the steps before it)
  __shared__ float hin_s[NS * 64];
  if (g.local) {
    const float* hp = hin + ((int64_t)q.s * g.batch + q.b) * NS * g.D + q.dc;
#pragma unroll
    for (int n = 0; n < NS; ++n) hin_s[n * 64 + q.lane] = hp[n * g.D];
  }
  issue_group(last / R);
  for (int j = last; j >= 0; --j) {
    // the group's copies have landed once every vector memory operation issued so far has
    // completed (the first sub-chunk taken from a group waits for them); that sub-chunk also
    // corrects the staged checkpoint of a zero-started segment in place, for the whole group
    if (j == last || (j % R) == R - 1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (g.local) {
        const float sck = lds_f32(NS * 64);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const float v = __builtin_fmaf(fast_exp2(a2[n] * sck), hin_s[n * 64 + q.lane], lds_f32(n * 64));
          stage[n * 64 + q.lane] = __builtin_bit_cast(uint32_t, v);
        }
      }
      if constexpr ((FX & kFront) != 0) {
        // the group's step sizes, once per staged step
        const float dbv = dbias_s[q.lane];
#pragma unroll
        for (int i = 0; i < KC; ++i)
          stage[kOffD + i * 64 + q.lane] = __builtin_bit_cast(uint32_t, step_size<FX>(lds_in(kOffD + i * 64), dbv));
      }
    }
    // inputs of the sub-chunk before, for the checkpoint advance of odd sub-chunks (the
    // first steps of the same group)
    float xa[K], da[K];
    if constexpr (R == 2) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        xa[i] = lds_in(kOffX + i * 64);
        da[i] = lds_dl(kOffD + i * 64);
      }
    }
    BWD_LOAD(0, j);
    float h0[NS];  // the checkpoint
#pragma unroll
    for (int n = 0; n < NS; ++n) h0[n] = lds_f32(n * 64);
    if (j % R == 0 && j > 0) {
      // the group's last sub-chunk: once its reads of the staging area have returned, the
      // next group's copies may overwrite it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_group(j / R - 1);
    }
    BWD_CHUNK(0, j);
  }
#undef BWD_LOAD
#undef BWD_CHUNK

#pragma unroll
  for (int n = 0; n < NS; ++n) part_a[(((int64_t)q.s * g.batch + q.b) * NS + n) * g.D + q.dc] = dacc[n];
  part_d[((int64_t)q.s * g.batch + q.b) * g.D + q.dc] = ddacc;
  if (q.s == 0 && dh0 != nullptr) {
#pragma unroll
    for (int n = 0; n < NS; ++n) dh0[chl + n] = mu[n];
  }
}

// ------------------------------------------------------------------ 5. partial sums
// dB[b][t][n] = sum_grp part[grp][b][t][n], dC from the second half of each row.
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* __restrict__ part, float* __restrict__ dB,
                                                     float* __restrict__ dC, int64_t rows /* batch * L */, int N,
                                                     int ngroups) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t V = 2 * (int64_t)N;
  if (idx >= rows * V) return;
  // the same sequential order, with a batch of loads in flight ahead of the adds
  constexpr int kAhead = 8;
  float acc = 0.0f;
  int gidx = 0;
  for (; gidx + kAhead <= ngroups; gidx += kAhead) {
    float v[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) v[k] = part[(int64_t)(gidx + k) * rows * V + idx];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) acc += v[k];
  }
  for (; gidx < ngroups; ++gidx) acc += part[(int64_t)gidx * rows * V + idx];
  const int64_t r = idx / V, j = idx - r * V;
  if (j < N) dB[r * N + j] = acc;
  else dC[r * N + (j - N)] = acc;
}

// Bias-gradient partials of the delta front end: part_db[s][b][d] = sum of ddelta[b][t][d] over
// segment s's steps, in time order (a thread per (s, b, d); adjacent threads read adjacent
// channels, so every row read is coalesced).
__global__ __launch_bounds__(256) void bwd_bias_partials(const float* __restrict__ ddelta, float* __restrict__ part_db,
                                                         int64_t batch, int64_t L, int64_t D, int64_t seg_len, int S) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (s * batch + b) * D + d
  if (idx >= (int64_t)S * batch * D) return;
  const int64_t d = idx % D, sb = idx / D, b = sb % batch, s = sb / batch;
  const int64_t t0 = s * seg_len, t1 = t0 + seg_len < L ? t0 + seg_len : L;
  const float* p = ddelta + (b * L + t0) * D + d;
  constexpr int kAhead = 8;
  float acc = 0.0f;
  int64_t t = t0;
  for (; t + kAhead <= t1; t += kAhead) {
    float v[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) v[k] = p[(t - t0 + k) * D];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) acc += v[k];
  }
  for (; t < t1; ++t) acc += p[(t - t0) * D];
  part_db[idx] = acc;
}

// dA[d][n] = sum_{s,b} part_a[s][b][n][d]; dD[d] = sum_{s,b} part_d[s][b][d]; with the delta
// front end, ddbias[d] = sum_{s,b} part_db[s][b][d].
__device__ __forceinline__ float sum_sb(const float* __restrict__ part, int64_t sb, int64_t stride) {
  // the sequential order, with a batch of loads in flight ahead of the adds
  constexpr int kAhead = 16;
  float acc = 0.0f;
  int64_t j = 0;
  for (; j + kAhead <= sb; j += kAhead) {
    float v[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) v[k] = part[(j + k) * stride];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) acc += v[k];
  }
  for (; j < sb; ++j) acc += part[j * stride];
  return acc;
}

__global__ __launch_bounds__(256) void bwd_reduce_ad(const float* __restrict__ part_a,
                                                     const float* __restrict__ part_d, float* __restrict__ dA,
                                                     float* __restrict__ dD, const float* __restrict__ part_db,
                                                     float* __restrict__ ddbias, int64_t sb /* S * batch */, int N,
                                                     int64_t D) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n * D + d
  if (idx >= (int64_t)N * D) return;
  const int64_t n = idx / D, d = idx - n * D;
  // the same sequential order, with a batch of loads in flight ahead of the adds
  constexpr int kAhead = 16;
  float acc = 0.0f;
  int64_t i = 0;
  for (; i + kAhead <= sb; i += kAhead) {
    float v[kAhead];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) v[k] = part_a[(i + k) * N * D + idx];
#pragma unroll
    for (int k = 0; k < kAhead; ++k) acc += v[k];
  }
  for (; i < sb; ++i) acc += part_a[i * N * D + idx];
  dA[d * N + n] = acc;
  if (n == 0 && dD != nullptr) {
    float ad = 0.0f;
    int64_t j = 0;
    for (; j + kAhead <= sb; j += kAhead) {
      float v[kAhead];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) v[k] = part_d[(j + k) * D + d];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) ad += v[k];
    }
    for (; j < sb; ++j) ad += part_d[j * D + d];
    dD[d] = ad;
  }
  // the bias sums on another thread than dD's where there is one (n = 1)
  if (n == (N > 1 ? 1 : 0) && ddbias != nullptr) ddbias[d] = sum_sb(part_db + d, sb, D);
}

// ------------------------------------------------------------------ host side
static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

BwdPlan plan_selective_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus) {
  BwdPlan bp{};
  bp.fwd = plan_selective(batch, seqlen, dim, dstate, num_cus);
  const int64_t S = bp.fwd.segments;
  const int K = bwd_k((int)dstate);
  bp.K = K;
  bp.KC = K * bwd_r((int)dstate);
  bp.nsub = (int)((bp.fwd.seg_len + bp.KC - 1) / bp.KC);
  const int64_t ngroups = (dim + 63) / 64;
  size_t off = align256(bp.fwd.ws_total);
  bp.off_mu = off;
  off = align256(off + (S > 1 ? (size_t)S * batch * dstate * dim * 4 : 0));
  bp.off_ckpt = off;
  off = align256(off + (size_t)S * bp.nsub * batch * (dstate + 1) * ((dim + 63) / 64) * 64 * 4);
  bp.off_bc = off;
  off = align256(off + (size_t)ngroups * batch * seqlen * 2 * dstate * 4);
  bp.off_pa = off;
  off = align256(off + (size_t)S * batch * dstate * dim * 4);
  bp.off_pd = off;
  off = align256(off + (size_t)S * batch * dim * 4);
  bp.off_pdb = off;  // bias-gradient partials (delta front end)
  off = align256(off + (size_t)S * batch * dim * 4);
  bp.ws_total = off;
  return bp;
}

template <int NS, bool BF16, int FX>
static hipError_t run_bwd(const BwdArgs& a, const BwdPlan& bp, hipStream_t stream) {
  unsigned char* ws = static_cast<unsigned char*>(a.fwd.workspace);
  const int S = bp.fwd.segments;
  BwdSeg g{};
  g.batch = a.fwd.batch;
  g.L = a.fwd.seqlen;
  g.D = a.fwd.dim;
  g.seg_len = bp.fwd.seg_len;
  g.S = S;
  g.ngroups = (int)((a.fwd.dim + 63) / 64);
  g.nsub = bp.nsub;
  g.K = bp.K;
  float* dsum = reinterpret_cast<float*>(ws + bp.fwd.ws_dsum);
  float* mu = reinterpret_cast<float*>(ws + bp.off_mu);
  float* ckpt = reinterpret_cast<float*>(ws + bp.off_ckpt);
  // entering states of zero-started segments: the forward plan's state slots
  g.local = (!a.states_ready && S > 1) ? 1 : 0;
  const float* hin = g.local ? reinterpret_cast<const float*>(ws + bp.fwd.ws_state) : nullptr;
  float* pbc = reinterpret_cast<float*>(ws + bp.off_bc);
  float* pa = reinterpret_cast<float*>(ws + bp.off_pa);
  float* pd = reinterpret_cast<float*>(ws + bp.off_pd);
  float* pdb = reinterpret_cast<float*>(ws + bp.off_pdb);
  const int64_t per_seg = (int64_t)g.ngroups * g.batch;
  hipError_t e;
  if (S > 1) {  // the segments' local folds are in mu (checkpoint pass)
    const int64_t nthr = g.batch * (int64_t)NS * g.D;
    hipLaunchKernelGGL(sel_bwd_carry, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream, a.fwd.A, a.dh_last,
                       mu, (const float*)dsum, g.batch, g.D, NS, S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(per_seg * S)), block(64);
  if (a.fwd.z != nullptr)
    hipLaunchKernelGGL((sel_bwd_kernel<NS, BF16, true, FX>), grid, block, 0, stream, a.fwd.x, a.fwd.delta, a.fwd.A,
                       a.fwd.B, a.fwd.C, a.fwd.Dsk, a.fwd.z, a.dy, a.dh_last, (const float*)mu, (const float*)ckpt, hin,
                       a.dx, a.ddelta, a.dz, pbc, pa, pd, a.dh0, a.fwd.delta_bias, g);
  else
    hipLaunchKernelGGL((sel_bwd_kernel<NS, BF16, false, FX>), grid, block, 0, stream, a.fwd.x, a.fwd.delta, a.fwd.A,
                       a.fwd.B, a.fwd.C, a.fwd.Dsk, a.fwd.z, a.dy, a.dh_last, (const float*)mu, (const float*)ckpt, hin,
                       a.dx, a.ddelta, a.dz, pbc, pa, pd, a.dh0, a.fwd.delta_bias, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((FX & kFront) != 0 && a.ddelta_bias != nullptr) {
    const int64_t nthr = (int64_t)S * g.batch * g.D;
    hipLaunchKernelGGL(bwd_bias_partials, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream,
                       (const float*)a.ddelta, pdb, g.batch, g.L, g.D, g.seg_len, S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t rows = g.batch * g.L;
  hipLaunchKernelGGL(bwd_reduce_bc, dim3((unsigned)((rows * 2 * NS + 255) / 256)), dim3(256), 0, stream,
                     (const float*)pbc, a.dB, a.dC, rows, NS, g.ngroups);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_ad, dim3((unsigned)(((int64_t)NS * g.D + 255) / 256)), dim3(256), 0, stream,
                     (const float*)pa, (const float*)pd, a.dA, a.dD, (const float*)pdb,
                     (FX & kFront) != 0 ? a.ddelta_bias : nullptr, (int64_t)S * g.batch, NS, g.D);
  return hipGetLastError();
}

template <bool BF16, int FX>
static hipError_t dispatch_bwd_n(const BwdArgs& a, const BwdPlan& bp, hipStream_t stream) {
  switch (a.fwd.dstate) {
    case 1: return run_bwd<1, BF16, FX>(a, bp, stream);
    case 2: return run_bwd<2, BF16, FX>(a, bp, stream);
    case 4: return run_bwd<4, BF16, FX>(a, bp, stream);
    case 8: return run_bwd<8, BF16, FX>(a, bp, stream);
    case 16: return run_bwd<16, BF16, FX>(a, bp, stream);
    case 32: return run_bwd<32, BF16, FX>(a, bp, stream);
    case 64: return run_bwd<64, BF16, FX>(a, bp, stream);
    default: return hipErrorInvalidValue;
  }
}

// the delta front end: none, bias only, or bias (optional) then softplus
template <bool BF16>
static hipError_t dispatch_bwd(const BwdArgs& a, const BwdPlan& bp, hipStream_t stream) {
  if (a.fwd.softplus) return dispatch_bwd_n<BF16, kFront | kSoftplus>(a, bp, stream);
  if (a.fwd.delta_bias != nullptr) return dispatch_bwd_n<BF16, kFront>(a, bp, stream);
  return dispatch_bwd_n<BF16, 0>(a, bp, stream);
}

hipError_t launch_selective_bwd(const BwdArgs& a, const BwdPlan& bp, hipStream_t stream) {
  // 1. the state before every K-th step and the segments' adjoint folds (the forward scan's
  //    checkpoint pass).  With several segments and no entering states kept by the forward
  //    call, every segment starts from zero and the same pass leaves the end states for the
  //    carry (no separate pass over the inputs for the entering states); with kept states
  //    the checkpoints start from them.
  const bool local = !a.states_ready && bp.fwd.segments > 1;
  hipError_t e = (a.states_ready || local) ? hipSuccess : launch_segment_states(a.fwd, bp.fwd, stream);
  if (e != hipSuccess) return e;
  unsigned char* ws = static_cast<unsigned char*>(a.fwd.workspace);
  e = launch_checkpoints(a.fwd, bp.fwd, reinterpret_cast<float*>(ws + bp.off_ckpt), ilog2c(bp.KC), bp.nsub, a.dy,
                         bp.fwd.segments > 1 ? reinterpret_cast<float*>(ws + bp.off_mu) : nullptr, local, stream);
  if (e != hipSuccess) return e;
  return a.fwd.bf16 ? dispatch_bwd<true>(a, bp, stream) : dispatch_bwd<false>(a, bp, stream);
}

}  // namespace sss
