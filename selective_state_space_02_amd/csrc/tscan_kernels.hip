// tscan_kernels.hip -- time-parallel selective scan for the (B,D,L) layout with 16 states.
//
// The recurrence h_t = a_t h_{t-1} + b_t (a_t = exp(dt_t A), b_t = dt_t u_t B_t, per state)
// is the associative scan of the pairs (a, b) under (a1,b1)(x)(a2,b2) = (a2 a1, a2 b1 + b2)
// («Mamba 选择性状态空间模型：亚二次复杂度大语言模型推理工程实践» §4.1; «Mamba与SSM状态空间模型：
// 一张摘要卡读完万页档案», 线性扫描算法).  Here one wave owns one channel (all 16 states) and
// walks its sequence in spans of 256 steps; inside a span the time axis is spread over the
// lanes:
//   lane l = 4 j + g : time chunk j (16 steps, j = 0..15) and state group g (states 4g..4g+3)
// Per span:
//   1. every lane loads and prepares 4 consecutive steps (dt, dt*u) of the span (lane l:
//      steps 4l..4l+3, i.e. chunk j's steps 4g..4g+3), shared through a per-wave LDS row;
//   2. fold: each lane runs its chunk's 16 steps from a zero state for its 4 states, keeping
//      every step's decay a and input b in registers, and forms the chunk's pair
//      (P, H) = (exp(A sum dt), end state from zero);
//   3. scan: the four chunks of a row of 16 lanes are combined with DPP row shifts (by 4 and
//      8 lanes, identity where no source lane exists); the rows' totals meet in LDS, folded
//      onto the span's carried-in state; each lane obtains the state at the start of its chunk;
//   4. readout: each lane reruns its 16 steps from that state with the cached (a, b) (one fma
//      per state and step) and forms its partial C_t . h_t; the chunk's four lanes exchange
//      the partials through LDS, and lane g finishes steps 4g..4g+3 (sum, D*u, gate, store),
//      which are the steps it loaded;
//   5. the last chunk's end state is the next span's carry (and h_last after the last span).
// Four waves (channels of one batch item and group) share the span's B/C tile in LDS, copied
// from the fp32 tile of bc_tile_kernel ([t][n][B C] per 32-step block) into [t][B0..15 C0..15].
// Inputs are read once, as contiguous runs of 512 bytes per wave and tensor.
// Padded steps (past L) take dt = 0 (a = 1, b = 0) and padded states A = B = C = 0, so
// neither changes a state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_plan.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int TS_T = 16;                 // steps per chunk
constexpr int TS_SPAN = 16 * TS_T;       // steps per span (16 chunks)
constexpr int TS_WAVES = 4;              // channels (waves) per workgroup
constexpr int TS_PART = TS_T + 4;        // padded row of a lane's readout partials

struct TsLds {
  float bc[TS_SPAN][32];                 // the span's B_t[0..15] then C_t[0..15]
  float dt[TS_WAVES][TS_SPAN];           // per channel: step sizes of the span
  float du[TS_WAVES][TS_SPAN];           // dt * u
  float part[TS_WAVES][64][TS_PART];     // per lane: readout partials of its chunk's steps
  float rowtot[TS_WAVES][4][4][8];       // [row][g][P0..3 H0..3]: in-row totals
  float carry[TS_WAVES][16];             // state at the span start
};

// softplus(r) = max(r, 0) + log1p(e), e = e^-|r|, log1p(e) = ln 2 log2(w) + (e - (w - 1)),
// w = fl(1 + e) in [1, 2]: the second term puts back the rounding of 1 + e
__device__ __forceinline__ float ts_softplus(float r) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(r) * kLog2e);
  const float w = 1.0f + e;
  return fmaf(__builtin_amdgcn_logf(w), kLn2, (r > 0.0f ? r : 0.0f) + (e - (w - 1.0f)));
}

__device__ __forceinline__ float ts_silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// x from the lane CTRL names (row shift); lanes without a source in their row get `old`
template <int CTRL>
__device__ __forceinline__ float ts_shift(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void wg_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// raw storage bits of element i (converted only where used, so a prefetch never waits)
template <bool BF16>
__device__ __forceinline__ uint32_t ts_bits(const void* p, int64_t i) {
  if (BF16) return ((const uint16_t*)p)[i];
  return ((const uint32_t*)p)[i];
}
template <bool BF16>
__device__ __forceinline__ float ts_cvt(uint32_t v) {
  return __uint_as_float(BF16 ? v << 16 : v);
}

template <bool BF16>
__device__ __forceinline__ void ts_store(void* p, int64_t i, float v) {
  if (BF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 w = {(__bf16)v, (__bf16)0.0f};
    ((uint16_t*)p)[i] = (uint16_t)(__builtin_bit_cast(uint32_t, w) & 0xffffu);
  } else {
    ((float*)p)[i] = v;
  }
}

// Grid: (ceil(rows_per_group / 4) * G, batch); 4 waves, one channel each.
template <bool BF16>
__global__ void __launch_bounds__(TS_WAVES * 64, 2) tscan_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) TsLds s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 2, g4 = lane & 3;
  const int bpg = (p.rows_per_group + TS_WAVES - 1) / TS_WAVES;
  const int grp = blockIdx.x / bpg;
  const int b = blockIdx.y;
  const int r_in = (blockIdx.x % bpg) * TS_WAVES + w;
  const bool chan_ok = r_in < p.rows_per_group;
  // a wave past the group's end repeats its last channel (same inputs, same results, same
  // places) so that every wave takes part in the workgroup barriers
  const int d = grp * p.rows_per_group + (chan_ok ? r_in : p.rows_per_group - 1);
  const int64_t L = p.L;
  const int64_t row = ((int64_t)b * p.dim + d) * L;      // first element of this channel's rows

  float A2[4], h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = 4 * g4 + i;
    A2[i] = n < p.N ? p.A[(int64_t)d * p.N + n] * kLog2e : 0.0f;
  }
  if (lane < 16) s.carry[w][lane] = (p.h0 && lane < p.N) ? p.h0[((int64_t)b * p.dim + d) * p.N + lane] : 0.0f;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const float* const tiles = p.bct + (int64_t)(b * p.G + grp) * p.nblk * (32 * 32);
  const int64_t nspan = (L + TS_SPAN - 1) / TS_SPAN;

  // Global loads of a span, issued one span ahead: the B/C tile (8 float4 per thread) and
  // this lane's 4 steps of delta, u, z (raw values).  Steps past the end load a clamped,
  // valid step (masked when used); tiles past the last block are zero.
  float4 pbc[8];
  uint32_t praw[4], pu[4], pz[4];
  auto prefetch = [&](int64_t t0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int idx = tid + 256 * r;                   // float4 index within the span (2048)
      const int t = idx >> 3, n = (idx & 7) * 2;
      const int64_t blk = (t0 >> 5) + (t >> 5);
      pbc[r] = blk < p.nblk ? *(const float4*)(tiles + (blk * 32 + (t & 31)) * 32 + n * 2)
                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = t0 + 4 * lane + q;
      const int64_t tc = t < L ? t : L - 1;          // clamped to a valid step
      praw[q] = ts_bits<BF16>(p.delta, row + tc);
      pu[q] = ts_bits<BF16>(p.u, row + tc);
      pz[q] = p.has_z ? ts_bits<BF16>(p.z, row + tc) : 0u;
    }
  };
  prefetch(0);

  for (int64_t sp = 0; sp < nspan; ++sp) {
    const int64_t t0 = sp * TS_SPAN;
    // ---- the span's B/C tile: 8 blocks of 32 steps, [t][n][B C] -> [t][B..][C..]
    wg_sync_lds();   // every wave is done with the previous span's tile
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int idx = tid + 256 * r;
      const int t = idx >> 3, n = (idx & 7) * 2;
      *(float2*)&s.bc[t][n] = make_float2(pbc[r].x, pbc[r].z);
      *(float2*)&s.bc[t][16 + n] = make_float2(pbc[r].y, pbc[r].w);
    }
    // ---- this lane's 4 steps: step sizes and dt * u
    float uu[4], zz[4];
    {
      float dtv[4], duv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t t = t0 + 4 * lane + q;
        uu[q] = ts_cvt<BF16>(pu[q]);
        zz[q] = ts_cvt<BF16>(pz[q]);
        const float rr = ts_cvt<BF16>(praw[q]) + bias;
        const float dt = t < L ? (p.softplus ? ts_softplus(rr) : rr) : 0.0f;
        dtv[q] = dt;
        duv[q] = dt * uu[q];
      }
      *(float4*)&s.dt[w][4 * lane] = make_float4(dtv[0], dtv[1], dtv[2], dtv[3]);
      *(float4*)&s.du[w][4 * lane] = make_float4(duv[0], duv[1], duv[2], duv[3]);
    }
    if (sp + 1 < nspan) prefetch(t0 + TS_SPAN);   // in flight while this span computes
    wg_sync_lds();   // the tile and every wave's dt / du rows are complete

    // ---- fold: this chunk's 16 steps from a zero state, (a, b) kept per step
    float a[TS_T][4], bx[TS_T][4], H[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float sdt = 0.0f;
#pragma unroll
    for (int q4 = 0; q4 < TS_T; q4 += 4) {
      const float4 d4 = *(const float4*)&s.dt[w][TS_T * j + q4];
      const float4 u4 = *(const float4*)&s.du[w][TS_T * j + q4];
      const float dq[4] = {d4.x, d4.y, d4.z, d4.w}, uq[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 B4 = *(const float4*)&s.bc[TS_T * j + q4 + q][4 * g4];
        const float Bv[4] = {B4.x, B4.y, B4.z, B4.w};
        sdt += dq[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[q4 + q][i] = __builtin_amdgcn_exp2f(dq[q] * A2[i]);
          bx[q4 + q][i] = uq[q] * Bv[i];
          H[i] = fmaf(a[q4 + q][i], H[i], bx[q4 + q][i]);
        }
      }
    }
    float P[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) P[i] = __builtin_amdgcn_exp2f(sdt * A2[i]);

    // ---- scan over the 4 chunks of this row: shifts by one and two chunks (4, 8 lanes)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float pp = ts_shift<0x114>(1.0f, P[i]), ph = ts_shift<0x114>(0.0f, H[i]);   // row_shr:4
      H[i] = fmaf(P[i], ph, H[i]);
      P[i] *= pp;
      pp = ts_shift<0x118>(1.0f, P[i]);                                           // row_shr:8
      ph = ts_shift<0x118>(0.0f, H[i]);
      H[i] = fmaf(P[i], ph, H[i]);
      P[i] *= pp;
    }
    // in-row exclusive prefix (identity for a row's first chunk), the rows' totals to LDS
    float eP[4], eH[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      eP[i] = ts_shift<0x114>(1.0f, P[i]);
      eH[i] = ts_shift<0x114>(0.0f, H[i]);
    }
    const int rw = j >> 2;
    if ((j & 3) == 3) {
      *(float4*)&s.rowtot[w][rw][g4][0] = make_float4(P[0], P[1], P[2], P[3]);
      *(float4*)&s.rowtot[w][rw][g4][4] = make_float4(H[0], H[1], H[2], H[3]);
    }
    wave_sync_lds();
    // state at the start of this row: the span's carry folded through the rows before it
    {
      const float4 c4 = *(const float4*)&s.carry[w][4 * g4];
      h[0] = c4.x; h[1] = c4.y; h[2] = c4.z; h[3] = c4.w;
    }
    for (int r = 0; r < rw; ++r) {
      const float4 tp = *(const float4*)&s.rowtot[w][r][g4][0];
      const float4 th = *(const float4*)&s.rowtot[w][r][g4][4];
      h[0] = fmaf(tp.x, h[0], th.x);
      h[1] = fmaf(tp.y, h[1], th.y);
      h[2] = fmaf(tp.z, h[2], th.z);
      h[3] = fmaf(tp.w, h[3], th.w);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = fmaf(eP[i], h[i], eH[i]);   // the start of this chunk

    // ---- readout: the chunk's steps again from its true start state
    float part[TS_T];
#pragma unroll
    for (int q = 0; q < TS_T; ++q) {
      const float4 C4 = *(const float4*)&s.bc[TS_T * j + q][16 + 4 * g4];
      const float Cv[4] = {C4.x, C4.y, C4.z, C4.w};
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = fmaf(a[q][i], h[i], bx[q][i]);
        acc = fmaf(Cv[i], h[i], acc);
      }
      part[q] = acc;
    }
    if (j == 15) *(float4*)&s.carry[w][4 * g4] = make_float4(h[0], h[1], h[2], h[3]);   // the next span's start
#pragma unroll
    for (int q = 0; q < TS_T; q += 4)
      *(float4*)&s.part[w][lane][q] = make_float4(part[q], part[q + 1], part[q + 2], part[q + 3]);
    wave_sync_lds();
    // steps 4 g4 .. 4 g4 + 3 of chunk j: the sum over the chunk's four state groups
    float ys[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const float4 v = *(const float4*)&s.part[w][4 * j + gg][4 * g4];
      ys[0] += v.x; ys[1] += v.y; ys[2] += v.z; ys[3] += v.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = t0 + 4 * lane + q;
      float yv = fmaf(Dd, uu[q], ys[q]);
      if (p.has_z) yv *= ts_silu(zz[q]);
      if (chan_ok && t < L) ts_store<BF16>(p.y, row + t, yv);
    }
  }
  // the last span's carry is the final state (padded steps leave it unchanged)
  wave_sync_lds();
  if (p.h_last && chan_ok && lane < p.N) p.h_last[((int64_t)b * p.dim + d) * p.N + lane] = s.carry[w][lane];
}

}  // namespace

int launch_tscan(const KParams& kp, bool bf16, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int bpg = (kp.rows_per_group + TS_WAVES - 1) / TS_WAVES;
  const dim3 grid(bpg * kp.G, kp.batch), block(TS_WAVES * 64);
  if (bf16) hipLaunchKernelGGL(tscan_kernel<true>, grid, block, 0, st, kp);
  else hipLaunchKernelGGL(tscan_kernel<false>, grid, block, 0, st, kp);
  return (int)hipGetLastError();
}

}  // namespace ssm
