// ssd_kernels.hip -- chunked (state-space-duality) form of the multi-head scan on MFMA.
//
// With one scalar A per head (the multi-head layout), the recurrence over a chunk of
// Q steps is a masked matrix product plus a carried state («AI底层架构的一场革命：Mamba如何用
// 「状态压缩」挑战Transformer的十年统治», section "Mamba-2：状态空间对偶性理论"; the SSD
// framework of «State Space Models 深度实战：从 S4 到 Mamba 的架构演进与 CUDA 优化» §4.1-§4.2).
// For head h, chunk steps t, s in [0, Q), cum_t = A * sum_{r<=t} dt_r, X_s = dt_s * u_s (P values):
//   y_t   = sum_{s<=t} exp(cum_t - cum_s) (C_t . B_s) X_s      intra-chunk: (L o C B^T) X
//         + exp(cum_t) C_t . H                                  from the state entering the chunk
//         + D u_t, times SiLU(z_t)
//   H'    = exp(cum_{Q-1}) H + sum_s exp(cum_{Q-1} - cum_s) B_s (x) X_s
// which is the recurrence h_t = exp(dt_t A) h_{t-1} + dt_t B_t u_t, regrouped exactly.
//
// The contractions run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  B and C are
// bfloat16 in memory, so they are exact operands.  The fp32 operands that feed the output
// -- the decayed C B^T, dt*u, its decayed copy and the state -- are split into a bfloat16
// high part and a bfloat16 remainder (x = hi + lo, |x - hi - lo| ~ 2^-17 |x|), and the
// products take hi*hi + hi*lo + lo*hi (decay x input), C*hi + C*lo (state) or
// B^T hi + B^T lo (chunk state), so the results keep about 16 bits instead of 8.  The
// state is carried in fp32.
//
// Work split: one workgroup (4 waves) walks the chunks of one (batch item, head, slice of
// PS positions) in order, with its slice of the state in registers; two workgroups fit on
// a CU.  Everything is computed transposed (rows = positions or states, columns = steps),
// so that each product's output tile is already in the layout its consumer reads:
//   G^T = B C^T              -> M^T = G^T o decay, stored [t][s] with 8-byte writes
//   Y^T = X^T M^T + H^T C^T  -> each lane holds 4 consecutive positions of one step: the
//                               row of y is written with 8-byte stores
//   H   = e^{cum_end} H + B^T (w X)  -> stored [p][n] with 8-byte writes for the next chunk
// The operands whose contraction runs over steps (X^T, B^T, w X) are read from their
// natural [step][.] layout with ds_read_b64_tr_b16, the gfx950 transposing LDS read: in
// each group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces addressed by
// lanes 4k + i/4 (k = 0..3), so with lane j addressing row k0 + j/4, columns 4(j%4)..+3
// of a [k][r] array, lane i gets column i of rows k0 .. k0+3.
//
// Optional input stage (CONV): u is SiLU of a causal depthwise convolution (width K <= 4,
// filter right-aligned in 4 taps) of the raw input x along time, per channel d = h P + p
// («AI底层架构的一场革命», section "Mamba Block：完整模块结构").  Each lane of a wave that
// stages u items convolves 2 channels x 4 consecutive steps of the wave's steps: it keeps
// its 2 filters in registers, loads the 7 raw inputs its 4 steps need (2 channels per
// 4-byte load; the carried state before t = 0), and leaves u in LDS, where the wave's own
// X = dt u staging and the output step's D u read it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_plan.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ float bf2f(uint32_t v16) { return __uint_as_float(v16 << 16); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats to a packed bf16 pair (round to nearest even), one instruction
__device__ __forceinline__ uint32_t pack_bf(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// a = ah + al, b = bh + bl (bf16 parts); hi = ah | bh << 16, lo = al | bl << 16
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf(a, b);
  lo = pack_bf(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// softplus(r) = max(r, 0) + log1p(e), e = 2^(-|r| log2 e), with log1p(e) taken as
// ln 2 * log2(w) + (e - (w - 1)), w = fl(1 + e) in [1, 2] (never overflows; w - 1 is exact).
// The second term puts back the rounding of 1 + e, which would otherwise be a relative error
// of up to 2^-24 / dt in every small step.
__device__ __forceinline__ float softplus_s(float r) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(r) * kLog2e);
  const float w = 1.0f + e;
  return fmaf(__builtin_amdgcn_logf(w), kLn2, (r > 0.0f ? r : 0.0f) + (e - (w - 1.0f)));
}

__device__ __forceinline__ float silu_s(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// x taken from another lane by a DPP pattern; lanes without a source (or in rows outside
// ROWS) read 0
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, true));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 from LDS (16-byte aligned)
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *(const bf16x8*)p; }

// Operand fragment of a [k][r] bf16 array in LDS (row stride RS elements, a multiple of 4):
// lane (l16, lq) receives rows k0 + 8 lq .. k0 + 8 lq + 7 of column r0 + l16.
template <int RS>
__device__ __forceinline__ bf16x8 ld8_tr(const uint16_t* base, int k0, int r0, int l16, int lq) {
  const uint16_t* p0 = base + (k0 + 8 * lq + (l16 >> 2)) * RS + r0 + 4 * (l16 & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * RS));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The same with the 32 contraction rows taken as two halves of 16, in the row order of
// two 16x16 MFMA results (rows 4 lq + r): lane (l16, lq) receives rows k0 + 4 lq .. +3
// and k0 + 16 + 4 lq .. +3 of column r0 + l16.
template <int RS>
__device__ __forceinline__ bf16x8 ld8_tr_halves(const uint16_t* base, int k0, int r0, int l16, int lq) {
  const uint16_t* p0 = base + (k0 + 4 * lq + (l16 >> 2)) * RS + r0 + 4 * (l16 & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 16 * RS));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Q = 64 steps per chunk, N states (32, 64 or 128), PS positions per workgroup (16 or 32).
// MFMA lane layout (16x16x32): A row = lane%16, k = 8*(lane/16)+i; B column = lane%16,
// k = 8*(lane/16)+i; D column = lane%16, rows 4*(lane/16)+r.
// A sequence cut into time segments of whole chunks runs an aggregate pass first (MODE 1:
// the state each segment before the last reaches from zero, and its decay e^{A sum dt},
// the chunk-carry form of the scan operator of «Mamba 选择性状态空间模型» §4.1); the
// main pass (MODE 0) folds the aggregates of the preceding segments into its initial state.
template <int N, int PS, bool ZOH, int MODE, bool CONV>
__global__ void __launch_bounds__(256, 2) ssd_kernel(KParams p) {
  constexpr int Q = 64;
  // Row strides (elements).  With 16-lane passes, a row stride of 16 B times an odd number
  // keeps the 16 rows of a 16-byte fragment read on distinct banks, and 7, 9 or 19 times
  // 16 B also keeps the 4 rows x 32 B of a transposing read apart.
  constexpr int BP = N == 32 ? 56 : N == 64 ? 72 : 152;   // sB [s][n]: read plainly and transposed
  constexpr int NP = N + 8;            // sH [p][n]: plain reads only
  constexpr int XP = PS == 16 ? 56 : 72;   // sX, sXW [s][hi p | lo p]: transposed reads
  static_assert(BP >= N && XP >= 2 * PS, "row strides");
  constexpr int NK = N / 32;           // 32-wide contraction steps over states
  constexpr int PT = PS / 16;          // 16-wide position tiles
  constexpr int NT = N / 16;           // 16-wide state tiles
  constexpr int NST = NT * PT;         // state tiles of the slice
  constexpr int SPW = (NST + 3) / 4;   // state tiles per wave (some waves may hold fewer)
  constexpr int NBI = Q * N / 8 / 256; // 16-byte B items per thread
  constexpr int NUI = Q * PS / 8;      // 16-byte u items of a chunk (threads below NUI own one)
  static_assert(NBI >= 1 && NUI <= 256, "items per thread");

  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * BP];         // B [s][n]
  __shared__ __attribute__((aligned(16))) uint16_t sX[Q * XP];         // dt*u [s][hi p | lo p]
  __shared__ __attribute__((aligned(16))) uint16_t sXW[Q * XP];        // e^{cum_end - cum_s} dt*u, same
  __shared__ __attribute__((aligned(16))) uint16_t sH[2][PS * NP];     // state [p][n], hi / lo
  __shared__ float sCum[4][Q];                                         // per wave: cum (log2 units)
  __shared__ float sDt[4][Q];                                          // per wave: step sizes
  constexpr int UP = PS + 4;                                           // row stride of sU
  __shared__ __attribute__((aligned(16))) float sU[CONV ? Q * UP : 4];   // u = SiLU(conv x) [s][p]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.  Renumber
  // them so that XCD k runs a contiguous range of (slice, head, batch): the heads of one
  // batch item that share a group's B and C chunks then read them from the same few L2s
  // (measured: HBM reads 2.3x -> 1.1x the algorithmic bytes on 80 heads of 64, 128 states).
  int pslice, hh, bz;
  {
    const int nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
    int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;
    pslice = id % nx;
    hh = (id / nx) % ny;
    bz = id / (nx * ny);
  }
  const int b = bz % p.batch, seg = bz / p.batch;   // batch item, time segment
  const int64_t L = p.L;
  const int64_t t_seg0 = (int64_t)seg * p.seg_len, t_seg1 = min(L, t_seg0 + p.seg_len);
  const int H = p.H, P = p.P, G = p.G;
  const int g = hh / p.heads_per_group;
  const int p0 = pslice * PS;
  const float A2 = p.A[hh] * kLog2e;
  const float biash = p.bias ? p.bias[hh] : 0.0f;
  // CONV: this lane's items, channels p0 + cpos, + 1 at steps cs0 .. cs0 + 3 of each chunk: the
  // wave stages the u items of steps [w CSW, (w + 1) CSW), CSW = 512 / PS (at PS = 16 waves 2
  // and 3 stage none); the filters (right-aligned in 4 taps) and biases stay in registers
  constexpr int CSW = 512 / PS;
  const int cpos = 2 * (lane % (PS / 2));
  const int cs0 = w * CSW + 4 * (lane / (PS / 2));
  const bool conv_lane = CONV && w * CSW < Q;
  float cwt[2][5] = {};
  if (CONV) {
    const int K = p.conv_k;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int64_t d = (int64_t)hh * p.P + p0 + cpos + q;
#pragma unroll
      for (int m = 0; m < 4; ++m) cwt[q][m] = m >= 4 - K ? p.conv_w[d * K + m - (4 - K)] : 0.0f;
      cwt[q][4] = p.conv_b ? p.conv_b[d] : 0.0f;
    }
  }

  // ---- the state: wave w holds state tiles k = w + 4 i (i < SPW, k < NST), tile k =
  //      (tn, tp) = (k / PT, k % PT); element (n, q) = (16 tn + 4 lq + r, 16 tp + l16)
  f32x4 hs[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = w + 4 * i, tn = k / PT, tp = k % PT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 16 * tn + 4 * lq + r, q = 16 * tp + l16;
      hs[i][r] = (MODE == 0 && k < NST && p.h0) ? p.h0[((int64_t)b * p.dim + (int64_t)hh * P + p0 + q) * N + n] : 0.0f;
    }
  }
  // segment aggregates: decays [seg][b][h], states [seg][b][h][slice][tile][lane][r]
  const int nslice = P / PS;
  auto agg_state = [&](int s2, int k) __attribute__((always_inline)) {
    return p.wsH + (((((int64_t)s2 * p.batch + b) * H + hh) * nslice + pslice) * NST + k) * 256 + 4 * lane;
  };
  if (MODE == 0) {
    for (int s2 = 0; s2 < seg; ++s2) {   // fold the preceding segments
      const float dec = p.wsP[((int64_t)s2 * p.batch + b) * H + hh];
#pragma unroll
      for (int i = 0; i < SPW; ++i) {
        const int k = w + 4 * i;
        if (k < NST) {
          const f32x4 a = *(const f32x4*)agg_state(s2, k);
#pragma unroll
          for (int r = 0; r < 4; ++r) hs[i][r] = fmaf(dec, hs[i][r], a[r]);
        }
      }
    }
  }
  auto store_state = [&]() __attribute__((always_inline)) {   // sH[q][n..n+3] = split(state): 8-byte writes
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w + 4 * i, tn = k / PT, tp = k % PT;
      if (k < NST) {
        uint32_t h0, l0, h1, l1;
        split2(hs[i][0], hs[i][1], h0, l0);
        split2(hs[i][2], hs[i][3], h1, l1);
        const int o = (16 * tp + l16) * NP + 16 * tn + 4 * lq;
        *(u32x2*)&sH[0][o] = (u32x2){h0, h1};
        *(u32x2*)&sH[1][o] = (u32x2){l0, l1};
      }
    }
  };
  if (MODE == 0) store_state();

  const uint16_t* const gB = (const uint16_t*)p.B;
  const uint16_t* const gC = (const uint16_t*)p.C;
  const uint16_t* const gU = (const uint16_t*)p.u;
  const uint16_t* const gDt = (const uint16_t*)p.delta;
  const uint16_t* const gZ = (const uint16_t*)(p.z ? p.z : p.u);
  uint16_t* const gY = (uint16_t*)p.y;
  const int64_t rowBC = (int64_t)G * N;          // elements between steps in B, C
  const int64_t rowX = (int64_t)H * P;           // elements between steps in u, z, y
  const int64_t colX = (int64_t)hh * P + p0;     // this slice's first position within a step

  // D of this lane's output positions: 4 per position tile
  float Dq[PT][4];
#pragma unroll
  for (int j = 0; j < PT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) Dq[j][r] = p.D ? p.D[colX + 16 * j + 4 * lq + r] : 0.0f;

  // ---- global loads of a chunk, issued one chunk ahead.  B items: (s, 8 states) per
  // 16 bytes, NBI per thread; u items: (s, 8 positions); C fragments: this wave's 16 steps,
  // 8 states per lane and contraction step; u and z of this lane's outputs; raw step size
  // of step lane.  Steps past the end load the last valid step (in-bounds, masked later).
  const int64_t last_chunk = ((L - 1) / Q) * Q;
  u32x4 pB[NBI] = {}, pC[NK] = {}, pU = {0u, 0u, 0u, 0u};
  uint32_t pXt[7] = {};   // CONV: raw x of this lane's 2 channels at steps cs0 - 3 .. cs0 + 3
  u32x2 pUo[PT] = {}, pZo[PT] = {};
  float pDelta = 0.0f;
  // per-lane element offsets of a chunk's loads from its first step, for full chunks and
  // for the last one (its steps past the end load its last valid step: in bounds, masked
  // later); only a uniform chunk base is computed per chunk
  struct Offs {
    uint32_t B[NBI], C, X, XZ, dt;
    int sx;   // step of this thread's u item within the chunk
  };
  auto offsets = [&](int nv) __attribute__((always_inline)) {
    Offs o;
#pragma unroll
    for (int k = 0; k < NBI; ++k) {
      const int it = tid + 256 * k, s = min(it / (N / 8), nv - 1), nb = (it % (N / 8)) * 8;
      o.B[k] = (uint32_t)(s * rowBC + nb);
    }
    const int tC = min(16 * w + l16, nv - 1);
    o.C = (uint32_t)(tC * rowBC + 8 * lq);
    o.sx = min(tid / (PS / 8), nv - 1);
    o.X = (uint32_t)(o.sx * rowX + (tid % (PS / 8)) * 8);
    o.XZ = (uint32_t)(tC * rowX + 4 * lq);
    o.dt = (uint32_t)(min(lane, nv - 1) * H);
    return o;
  };
  const Offs ofull = offsets(Q), olast = offsets((int)(L - last_chunk));
  auto prefetch = [&, gB, gC, gU, gDt, gZ, rowBC, rowX, colX, last_chunk, ofull, olast](int64_t tc)
                      __attribute__((always_inline)) {
    const bool last = tc == last_chunk;
    const int64_t row0 = (int64_t)b * L + tc;    // uniform
    const uint16_t* const bB = gB + row0 * rowBC + (int64_t)g * N;
#pragma unroll
    for (int k = 0; k < NBI; ++k) pB[k] = *(const u32x4*)(bB + (last ? olast.B[k] : ofull.B[k]));
    const uint16_t* const bC = gC + row0 * rowBC + (int64_t)g * N + (last ? olast.C : ofull.C);
    const uint16_t* const bX = gU + row0 * rowX + colX;
    if (tid < NUI && !CONV) pU = *(const u32x4*)(bX + (last ? olast.X : ofull.X));
    if (conv_lane) {   // steps before t = 0 re-read step 0, past the end the last step (replaced / masked)
      const int nv = last ? (int)(L - last_chunk) : Q;
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        int st = cs0 - 3 + i;
        if (tc + st < 0) st = (int)-tc;
        if (st > nv - 1) st = nv - 1;
        pXt[i] = *(const uint32_t*)(bX + (int64_t)st * rowX + cpos);
      }
    }
    if (MODE == 0) {   // C and the outputs' u and z: the main pass only
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) pC[kk] = *(const u32x4*)(bC + 32 * kk);
      const uint32_t oxz = last ? olast.XZ : ofull.XZ;
      const uint16_t* const bZ = gZ + row0 * rowX + colX;
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        if (!CONV) pUo[j] = *(const u32x2*)(bX + oxz + 16 * j);
        pZo[j] = *(const u32x2*)(bZ + oxz + 16 * j);
      }
    }
    pDelta = bf2f(gDt[row0 * H + hh + (last ? olast.dt : ofull.dt)]);
  };
  const int64_t seg_last = ((t_seg1 - 1) / Q) * Q;   // first step of the segment's last chunk
  prefetch(t_seg0);
  float lsum = 0.0f;   // aggregate pass: log2 of the segment's decay

  for (int64_t t0 = t_seg0; t0 < t_seg1; t0 += Q) {
    const int nval = (int)min((int64_t)Q, L - t0);
    // ===== stage: B rows; this wave's step sizes and prefix sums; X and w X ===============
#pragma unroll
    for (int k = 0; k < NBI; ++k) {
      const int it = tid + 256 * k, s = it / (N / 8), nb = (it % (N / 8)) * 8;
      *(u32x4*)&sB[s * BP + nb] = pB[k];
    }
    u32x4 cC[NK];
    u32x2 cUo[PT], cZo[PT];
    if (MODE == 0) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) cC[kk] = pC[kk];
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        cUo[j] = pUo[j];
        cZo[j] = pZo[j];
      }
    }
    const u32x4 cU = pU;
    if (conv_lane) {   // u of this lane's 2 channels x 4 steps, into LDS for the wave's X staging
      float xw[2][7];
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        xw[0][i] = bf2f(pXt[i] & 0xffffu);
        xw[1][i] = bf2f(pXt[i] >> 16);
      }
      if (t0 + cs0 < 3) {   // steps before t = 0: the carried raw inputs (or zeros)
        const int K1 = p.conv_k - 1;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int64_t tt = t0 + cs0 - 3 + i;
          if (tt < 0) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int64_t d = (int64_t)hh * P + p0 + cpos + q;
              xw[q][i] = (p.conv_sin && tt >= -(int64_t)K1) ? p.conv_sin[((int64_t)b * p.dim + d) * K1 + K1 + tt]
                                                            : 0.0f;
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float uq[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float c = cwt[q][4];
#pragma unroll
          for (int m = 0; m < 4; ++m) c = fmaf(cwt[q][m], xw[q][j + m], c);
          uq[q] = silu_s(c);
        }
        *(float2*)&sU[(cs0 + j) * UP + cpos] = make_float2(uq[0], uq[1]);
      }
    }
    {   // every wave computes the chunk's step sizes and prefix sums itself (no barrier)
      float dt = 0.0f;
      if (lane < nval) {
        const float r = pDelta + biash;
        dt = p.softplus ? softplus_s(r) : r;
      }
      // inclusive prefix sum over the 64 lanes with DPP (no LDS round trips): shifts within
      // rows of 16, then the last lane of row 0 / rows 0-1 broadcast into the rows above
      float c = dt;
      c += dpp_f<0x111, 0xf>(c);   // row_shr:1
      c += dpp_f<0x112, 0xf>(c);   // row_shr:2
      c += dpp_f<0x114, 0xf>(c);   // row_shr:4
      c += dpp_f<0x118, 0xf>(c);   // row_shr:8
      c += dpp_f<0x142, 0xa>(c);   // row_bcast:15 into rows 1 and 3
      c += dpp_f<0x143, 0xc>(c);   // row_bcast:31 into rows 2 and 3
      sDt[w][lane] = dt;
      sCum[w][lane] = c * A2;     // log2 of the decay from the chunk start through step lane
    }
    // the next chunk's loads fly while this one computes (the last chunk re-reads itself)
    prefetch(min(t0 + Q, seg_last));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const float cum_end = sCum[w][Q - 1];
    lsum += cum_end;
    if (tid < NUI) {   // X = dt u and w X of one u item, split into hi / lo
      const int s = tid / (PS / 8), qb = (tid % (PS / 8)) * 8;
      float dts = sDt[w][s];
      if (ZOH) {   // exact hold per head: dt -> expm1(x)/x * dt, x = dt*A
        const float y = dts * A2, x = y * kLn2;
        const float poly = fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f), 1.0f);
        dts *= fabsf(x) < 0.125f ? poly : (__builtin_amdgcn_exp2f(y) - 1.0f) * __builtin_amdgcn_rcpf(x);
      }
      const float ws = __builtin_amdgcn_exp2f(cum_end - sCum[w][s]);
      float uv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uv[2 * i] = bf2f(cU[i] & 0xffffu);
        uv[2 * i + 1] = bf2f(cU[i] >> 16);
      }
      if (CONV) {   // u from this wave's conv lanes
        const f32x4 lo = *(const f32x4*)&sU[s * UP + qb], hi = *(const f32x4*)&sU[s * UP + qb + 4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uv[i] = lo[i];
          uv[4 + i] = hi[i];
        }
      }
      uint32_t xh[4], xl[4], wh[4], wl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = dts * uv[2 * i], x1 = dts * uv[2 * i + 1];
        split2(x0, x1, xh[i], xl[i]);
        split2(x0 * ws, x1 * ws, wh[i], wl[i]);
      }
      if (MODE == 0) {
        *(u32x4*)&sX[s * XP + qb] = (u32x4){xh[0], xh[1], xh[2], xh[3]};
        *(u32x4*)&sX[s * XP + PS + qb] = (u32x4){xl[0], xl[1], xl[2], xl[3]};
      }
      *(u32x4*)&sXW[s * XP + qb] = (u32x4){wh[0], wh[1], wh[2], wh[3]};
      *(u32x4*)&sXW[s * XP + PS + qb] = (u32x4){wl[0], wl[1], wl[2], wl[3]};
    }
    __syncthreads();   // sB, sX, sXW of this chunk and sH of the previous one are complete

    // ===== wave w: output steps t in [16w, 16w+16) =========================================
    const int ks = 32 * ((w + 2) / 2);   // contraction range over steps covering s <= 16w+15
    if (MODE == 0) {
      // M^T = (B C^T) o decay for the step tiles i <= w of this wave's column tile (zeros
      // for i > w inside the range ks), kept in registers as hi / lo bf16 pairs in the
      // layout of the MFMA result (lane: step t, steps s = 16 i + 4 lq + r), which is the
      // operand layout of the next product with its contraction rows taken in two halves
      const int t = 16 * w + l16;
      const float cum_t = sCum[w][t];
      u32x2 mh[4], ml[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mh[i] = (u32x2){0u, 0u};
        ml[i] = (u32x2){0u, 0u};
        if (16 * i >= ks) continue;
        uint32_t h0 = 0, l0 = 0, h1 = 0, l1 = 0;
        if (i <= w) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NK; ++kk)
            acc = mfma(ld8(&sB[(16 * i + l16) * BP + 32 * kk + 8 * lq]), __builtin_bit_cast(bf16x8, cC[kk]), acc);
          // the decay of every lane, then a select: masked lanes (s > t) may hold inf, never used
          const f32x4 cs = *(const f32x4*)&sCum[w][16 * i + 4 * lq];
          float m[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(cum_t - cs[r]);
            m[r] = 16 * i + 4 * lq + r <= t ? acc[r] * e : 0.0f;
          }
          split2(m[0], m[1], h0, l0);
          split2(m[2], m[3], h1, l1);
        }
        mh[i] = (u32x2){h0, h1};
        ml[i] = (u32x2){l0, l1};
      }

      // Y^T = X^T M^T + H^T C^T per position tile; lane: step t, positions 16 j + 4 lq + r
      const float et = __builtin_amdgcn_exp2f(cum_t);
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        f32x4 yd = {0.f, 0.f, 0.f, 0.f}, yo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {   // steps s in [32 kc, 32 kc + 32): M tiles 2 kc, 2 kc + 1
          if (32 * kc >= ks) continue;     // uniform
          const bf16x8 xa = ld8_tr_halves<XP>(sX, 32 * kc, 16 * j, l16, lq);
          const bf16x8 xl = ld8_tr_halves<XP>(sX, 32 * kc, PS + 16 * j, l16, lq);
          const bf16x8 mb = __builtin_bit_cast(bf16x8, (u32x4){mh[2 * kc][0], mh[2 * kc][1], mh[2 * kc + 1][0], mh[2 * kc + 1][1]});
          const bf16x8 mlo = __builtin_bit_cast(bf16x8, (u32x4){ml[2 * kc][0], ml[2 * kc][1], ml[2 * kc + 1][0], ml[2 * kc + 1][1]});
          yd = mfma(xa, mb, yd);
          yd = mfma(xa, mlo, yd);
          yd = mfma(xl, mb, yd);
        }
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const bf16x8 c = __builtin_bit_cast(bf16x8, cC[kk]);
          yo = mfma(ld8(&sH[0][(16 * j + l16) * NP + 32 * kk + 8 * lq]), c, yo);
          yo = mfma(ld8(&sH[1][(16 * j + l16) * NP + 32 * kk + 8 * lq]), c, yo);
        }
        // y = Yd + e^{cum_t} Yo + D u, gated: 4 consecutive positions of step t
        const uint32_t u01 = cUo[j][0], u23 = cUo[j][1], z01 = cZo[j][0], z23 = cZo[j][1];
        float uv[4] = {bf2f(u01 & 0xffffu), bf2f(u01 >> 16), bf2f(u23 & 0xffffu), bf2f(u23 >> 16)};
        if (CONV) {
          const f32x4 uc = *(const f32x4*)&sU[t * UP + 16 * j + 4 * lq];
#pragma unroll
          for (int r = 0; r < 4; ++r) uv[r] = uc[r];
        }
        const float zv[4] = {bf2f(z01 & 0xffffu), bf2f(z01 >> 16), bf2f(z23 & 0xffffu), bf2f(z23 >> 16)};
        float yv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          yv[r] = fmaf(et, yo[r], yd[r]) + Dq[j][r] * uv[r];
          if (p.z) yv[r] *= silu_s(zv[r]);
        }
        if (t < nval) {
          const u32x2 o = {pack_bf(yv[0], yv[1]), pack_bf(yv[2], yv[3])};
          // plain stores: the L2 merges the 32-byte pieces of a line before writing it back
          // (streaming stores wrote 1.4x the bytes of y)
          *(u32x2*)(gY + ((int64_t)b * L + t0 + t) * rowX + colX + 16 * j + 4 * lq) = o;
        }
      }
    }
    // ===== the chunk's state contribution S = B^T (w X), then the new state ================
    const float dec = __builtin_amdgcn_exp2f(cum_end);
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w + 4 * i, tn = k / PT, tp = k % PT;
      if (k < NST) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Q; kk += 32) {
          const bf16x8 a = ld8_tr<BP>(sB, kk, 16 * tn, l16, lq);
          sacc = mfma(a, ld8_tr<XP>(sXW, kk, 16 * tp, l16, lq), sacc);
          sacc = mfma(a, ld8_tr<XP>(sXW, kk, PS + 16 * tp, l16, lq), sacc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[i][r] = fmaf(dec, hs[i][r], sacc[r]);
      }
    }
    __syncthreads();   // every wave is done with this chunk's sB, sX, sXW and the old sH
    if (MODE == 0) store_state();
  }
  if (MODE == 1) {   // the segment's aggregate: its zero-start end state and its decay
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w + 4 * i;
      if (k < NST) *(f32x4*)agg_state(seg, k) = hs[i];
    }
    if (pslice == 0 && tid == 0) p.wsP[((int64_t)seg * p.batch + b) * H + hh] = __builtin_amdgcn_exp2f(lsum);
    return;
  }
  // ---- the last K-1 raw inputs of this slice's channels, for a continuing call
  if (CONV && p.conv_sout && seg == p.nseg - 1) {
    const int K1 = p.conv_k - 1;
    if (tid < PS * K1) {
      const int q = tid / K1, j = tid % K1;
      const int64_t d = (int64_t)hh * P + p0 + q, tt = L - K1 + j;
      float v = 0.0f;
      if (tt >= 0) v = bf2f(gU[((int64_t)b * L + tt) * rowX + colX + q]);
      else if (p.conv_sin) v = p.conv_sin[((int64_t)b * p.dim + d) * K1 + K1 + tt];
      p.conv_sout[((int64_t)b * p.dim + d) * K1 + j] = v;
    }
  }
  // ---- final state
  if (p.h_last && seg == p.nseg - 1) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w + 4 * i, tn = k / PT, tp = k % PT;
      if (k < NST) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 16 * tn + 4 * lq + r, q = 16 * tp + l16;
          p.h_last[((int64_t)b * p.dim + colX + q) * N + n] = hs[i][r];
        }
      }
    }
  }
}

template <int N, int PS, bool ZOH, bool CONV>
int launch_ps_z(const KParams& kp, hipStream_t st) {
  if (kp.nseg > 1) {   // aggregates of the segments before the last
    hipLaunchKernelGGL((ssd_kernel<N, PS, ZOH, 1, CONV>), dim3(kp.P / PS, kp.H, kp.batch * (kp.nseg - 1)), dim3(256),
                       0, st, kp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  hipLaunchKernelGGL((ssd_kernel<N, PS, ZOH, 0, CONV>), dim3(kp.P / PS, kp.H, kp.batch * kp.nseg), dim3(256), 0, st,
                     kp);
  return (int)hipGetLastError();
}

template <int N, int PS>
int launch_ps(const KParams& kp, int zoh, hipStream_t st) {
  if (kp.conv_k > 0)
    return zoh ? launch_ps_z<N, PS, true, true>(kp, st) : launch_ps_z<N, PS, false, true>(kp, st);
  return zoh ? launch_ps_z<N, PS, true, false>(kp, st) : launch_ps_z<N, PS, false, false>(kp, st);
}

template <int N>
int launch_n(const KParams& kp, int ps, int zoh, hipStream_t st) {
  switch (ps) {
    case 32: return launch_ps<N, 32>(kp, zoh, st);
    case 16: return launch_ps<N, 16>(kp, zoh, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

// N in {32, 64, 128}; ps (positions per workgroup) in {16, 32} and divides P.
int launch_ssd(const KParams& kp, int ps, int zoh, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  switch (kp.N) {
    case 32: return launch_n<32>(kp, ps, zoh, st);
    case 64: return launch_n<64>(kp, ps, zoh, st);
    case 128: return launch_n<128>(kp, ps, zoh, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace ssm
