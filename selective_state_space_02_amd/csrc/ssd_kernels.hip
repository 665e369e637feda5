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
// The three contractions (C B^T over states, (L o C B^T) X over steps, C H over
// states, B^T X over steps) run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
// B and C are bfloat16 in memory, so they are exact operands.  The fp32 operands
// that feed the output -- the decayed C B^T, dt*u and the state -- are split into a
// bfloat16 high part and a bfloat16 remainder (x = hi + lo, |x - hi - lo| ~ 2^-17 |x|),
// and the products take hi*hi + hi*lo + lo*hi (decay x input), C*hi + C*lo (state)
// or B^T hi + B^T lo (chunk state), so the results keep about 16 bits instead of 8.
// The state is carried in fp32.  One workgroup (4 waves) walks the chunks of one (batch, head,
// slice of PS positions) in order with the state in registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_plan.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }
__device__ __forceinline__ uint16_t f2bf(float v) {
  const bf16 b = (bf16)v;
  return __builtin_bit_cast(uint16_t, b);
}
// x = bf16 hi + bf16 lo
__device__ __forceinline__ void split_bf(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

__device__ __forceinline__ float softplus_s(float r) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(r) * kLog2e);
  const float w = 1.0f + e;
  const float err = e - (w - 1.0f);
  return (r > 0.0f ? r : 0.0f) + fmaf(__builtin_amdgcn_logf(w), kLn2, err);
}

__device__ __forceinline__ float silu_s(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 from LDS (16-byte aligned)
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *(const bf16x8*)p; }

// Q = 64 steps per chunk, N states (multiple of 32, <= 128), PS positions per workgroup
// (16, 32 or 64).  MFMA lane layout (16x16x32): A row = lane%16, k = 8*(lane/16)+i;
// B column = lane%16, k = 8*(lane/16)+i; D column = lane%16, rows 4*(lane/16)+r.
template <int N, int PS, bool ZOH>
__global__ void __launch_bounds__(256) ssd_kernel(KParams p) {
  constexpr int Q = 64;
  constexpr int NP = N + 8;        // padded LDS row of N bf16
  constexpr int QP = Q + 8;        // padded LDS row of Q bf16
  constexpr int UP = PS + 8;       // padded LDS row of PS bf16
  constexpr int NT = N / 16, PT = PS / 16;          // 16-wide tiles along states / positions
  constexpr int SPW = (NT * PT) / 4;                // state tiles per wave
  static_assert((NT * PT) % 4 == 0, "state tiles must split over 4 waves");

  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * NP];     // C [t][n]
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * NP];     // B [s][n]
  __shared__ __attribute__((aligned(16))) uint16_t sBt[N * QP];    // B^T [n][s]
  __shared__ __attribute__((aligned(16))) uint16_t sXt[PS * QP];   // (dt*u)^T [p][s], high part
  __shared__ __attribute__((aligned(16))) uint16_t sXtl[PS * QP];  // its remainder
  __shared__ __attribute__((aligned(16))) uint16_t sXWt[PS * QP];  // (w*dt*u)^T [p][s], w_s = exp(cum_end - cum_s)
  __shared__ __attribute__((aligned(16))) uint16_t sXWtl[PS * QP]; // its remainder
  __shared__ __attribute__((aligned(16))) uint16_t sM[4][16 * QP]; // per wave: its 16 rows of (L o C B^T), high
  __shared__ __attribute__((aligned(16))) uint16_t sMl[4][16 * QP];// remainder
  __shared__ __attribute__((aligned(16))) uint16_t sHt[PS * NP];   // state^T [p][n] (bf16 operand copy), high
  __shared__ __attribute__((aligned(16))) uint16_t sHtl[PS * NP];  // remainder
  __shared__ __attribute__((aligned(16))) uint16_t sU[Q * UP];    // u [t][p] (for the D*u skip)
  __shared__ __attribute__((aligned(16))) uint16_t sZ[Q * UP];    // z [t][p] (for the gate)
  __shared__ float sDt[Q], sCum[Q];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int pslice = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
  const int64_t L = p.L;
  const int H = p.H, P = p.P, G = p.G;
  const int g = hh / p.heads_per_group;
  const int p0 = pslice * PS;
  const float A2 = p.A[hh] * kLog2e;
  const float biash = p.bias ? p.bias[hh] : 0.0f;

  // ---- the state: wave w holds state tiles k = w*SPW + i, tile k = (tn, tp) = (k / PT, k % PT);
  //      element (n, q) = (16 tn + 4 lq + r, 16 tp + l16) of the (N x PS) state of this slice
  f32x4 hs[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = w * SPW + i, tn = k / PT, tp = k % PT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 16 * tn + 4 * lq + r, q = 16 * tp + l16;
      hs[i][r] = p.h0 ? p.h0[((int64_t)b * p.dim + (int64_t)hh * P + p0 + q) * N + n] : 0.0f;
    }
  }
  auto store_state_operand = [&]() {    // sHt[q][n] = bf16(state)
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w * SPW + i, tn = k / PT, tp = k % PT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * tp + l16) * NP + 16 * tn + 4 * lq + r;
        split_bf(hs[i][r], sHt[o], sHtl[o]);
      }
    }
  };
  store_state_operand();

  const uint16_t* const gB = (const uint16_t*)p.B;
  const uint16_t* const gC = (const uint16_t*)p.C;
  const uint16_t* const gU = (const uint16_t*)p.u;
  const uint16_t* const gDt = (const uint16_t*)p.delta;
  const uint16_t* const gZ = (const uint16_t*)(p.z ? p.z : p.u);
  uint16_t* const gY = (uint16_t*)p.y;

  // ---- global loads of the next chunk, issued while the current one computes.  Every
  // thread owns fixed items: B/C item k = (s, 8 states), u/z item k = (s, 8 positions),
  // with s = (tid + 256 k) % Q.  Rows past the end of the sequence load the last valid
  // row (an in-bounds address) and are zeroed when staged.
  constexpr int NBI = Q * (N / 8) / 256, NUI = Q * (PS / 8) / 256;
  static_assert(NBI >= 1 && NUI >= 1, "items per thread");
  const int64_t last_chunk = ((L - 1) / Q) * Q;
  uint4 pB[NBI], pC[NBI], pU[NUI], pZ[NUI];
  float pDelta;
  auto prefetch = [&](int64_t tc) {
    const int nv = (int)min((int64_t)Q, L - tc);
#pragma unroll
    for (int k = 0; k < NBI; ++k) {
      const int it = tid + 256 * k, s = min(it % Q, nv - 1), nb = (it / Q) * 8;
      const int64_t gi = (((int64_t)b * L + tc + s) * G + g) * N + nb;
      pB[k] = *(const uint4*)(gB + gi);
      pC[k] = *(const uint4*)(gC + gi);
    }
#pragma unroll
    for (int k = 0; k < NUI; ++k) {
      const int it = tid + 256 * k, s = min(it % Q, nv - 1), qb = (it / Q) * 8;
      const int64_t gi = (((int64_t)b * L + tc + s) * H + hh) * P + p0 + qb;
      pU[k] = *(const uint4*)(gU + gi);
      pZ[k] = *(const uint4*)(gZ + gi);
    }
    pDelta = bf2f(gDt[((int64_t)b * L + tc + min(lane, nv - 1)) * H + hh]);
  };
  prefetch(0);

  for (int64_t t0 = 0; t0 < L; t0 += Q) {
    const int nval = (int)min((int64_t)Q, L - t0);
    // ================= phase 1: stage B, B^T, C, u, z, dt, cumulative decay, X ============
    // (raw 16-bit words, not bf16 vector elements, so each element is addressed explicitly)
#pragma unroll
    for (int k = 0; k < NBI; ++k) {
      const int it = tid + 256 * k, s = it % Q, nb = (it / Q) * 8;
      const bool ok = s < nval;
      const uint4 bv = ok ? pB[k] : make_uint4(0u, 0u, 0u, 0u);
      const uint4 cv = ok ? pC[k] : make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)&sB[s * NP + nb] = bv;
      *(uint4*)&sC[s * NP + nb] = cv;
      const uint32_t wv[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sBt[(nb + 2 * i) * QP + s] = (uint16_t)(wv[i] & 0xffffu);
        sBt[(nb + 2 * i + 1) * QP + s] = (uint16_t)(wv[i] >> 16);
      }
    }
#pragma unroll
    for (int k = 0; k < NUI; ++k) {
      const int it = tid + 256 * k, s = it % Q, qb = (it / Q) * 8;
      const bool ok = s < nval;
      *(uint4*)&sU[s * UP + qb] = ok ? pU[k] : make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)&sZ[s * UP + qb] = ok ? pZ[k] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (w == 0) {   // step sizes and their inclusive prefix sum (times A, log2 units)
      float dt = 0.0f;
      if (lane < nval) {
        const float r = pDelta + biash;
        dt = p.softplus ? softplus_s(r) : r;
      }
      float c = dt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float v = __shfl_up(c, o);
        if (lane >= o) c += v;
      }
      sDt[lane] = dt;
      sCum[lane] = c * A2;        // log2 of the decay from the chunk start through step lane
    }
    __syncthreads();
    const float cum_end = sCum[Q - 1];
    // X^T and (w X)^T from this thread's u items (zero past the end)
#pragma unroll
    for (int k = 0; k < NUI; ++k) {
      const int it = tid + 256 * k, s = it % Q, qb = (it / Q) * 8;
      float dts = sDt[s];
      if (ZOH) {   // exact hold per head: dt -> expm1(x)/x * dt, x = dt*A
        const float y = dts * A2, x = y * kLn2;
        const float poly = fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f), 1.0f);
        dts *= fabsf(x) < 0.125f ? poly : (__builtin_amdgcn_exp2f(y) - 1.0f) * __builtin_amdgcn_rcpf(x);
      }
      const float ws = __builtin_amdgcn_exp2f(cum_end - sCum[s]);
      const uint4 uv = s < nval ? pU[k] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t wu[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = dts * bf2f((uint16_t)((i & 1) ? (wu[i >> 1] >> 16) : (wu[i >> 1] & 0xffffu)));
        split_bf(x, sXt[(qb + i) * QP + s], sXtl[(qb + i) * QP + s]);
        split_bf(x * ws, sXWt[(qb + i) * QP + s], sXWtl[(qb + i) * QP + s]);
      }
    }
    __syncthreads();
    // next chunk's loads fly while this one computes (the last chunk re-reads itself)
    prefetch(min(t0 + Q, last_chunk));

    // ================= phase 2a: wave w owns output rows t in [16w, 16w+16) ===============
    {
      const int tr = 16 * w;
      // G = C B^T for column tiles j <= w, masked and decayed into this wave's rows of M
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j > w) {   // zero tile (s > t) inside the K range that Y_diag reads
          if (j < 2 * ((w + 2) / 2)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sM[w][(4 * lq + r) * QP + 16 * j + l16] = sMl[w][(4 * lq + r) * QP + 16 * j + l16] = 0;
          }
          continue;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < N; kk += 32) {
          const bf16x8 a = ld8(&sC[(tr + l16) * NP + kk + 8 * lq]);
          const bf16x8 bb = ld8(&sB[(16 * j + l16) * NP + kk + 8 * lq]);
          acc = mfma(a, bb, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tr + 4 * lq + r, s = 16 * j + l16;
          const float m = s <= t ? acc[r] * __builtin_amdgcn_exp2f(sCum[t] - sCum[s]) : 0.0f;
          split_bf(m, sM[w][(4 * lq + r) * QP + s], sMl[w][(4 * lq + r) * QP + s]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Y = M X (steps s <= t) and C H (from the entering state), per 16-position tile
      const int ks = 32 * ((w + 2) / 2);                     // K range covering s <= 16w+15
#pragma unroll
      for (int tp = 0; tp < PT; ++tp) {
        f32x4 yd = {0.f, 0.f, 0.f, 0.f}, yo = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < ks; kk += 32) {
          const bf16x8 a = ld8(&sM[w][l16 * QP + kk + 8 * lq]);
          const bf16x8 al = ld8(&sMl[w][l16 * QP + kk + 8 * lq]);
          const bf16x8 bb = ld8(&sXt[(16 * tp + l16) * QP + kk + 8 * lq]);
          const bf16x8 bl = ld8(&sXtl[(16 * tp + l16) * QP + kk + 8 * lq]);
          yd = mfma(a, bb, yd);
          yd = mfma(a, bl, yd);
          yd = mfma(al, bb, yd);
        }
#pragma unroll
        for (int kk = 0; kk < N; kk += 32) {
          const bf16x8 a = ld8(&sC[(tr + l16) * NP + kk + 8 * lq]);
          const bf16x8 bb = ld8(&sHt[(16 * tp + l16) * NP + kk + 8 * lq]);
          const bf16x8 bl = ld8(&sHtl[(16 * tp + l16) * NP + kk + 8 * lq]);
          yo = mfma(a, bb, yo);
          yo = mfma(a, bl, yo);
        }
        // epilogue: y = Yd + e^{cum_t} Yo + D u, gated; column q = 16 tp + l16, rows t = tr + 4 lq + r
        const int q = 16 * tp + l16;
        const float Dq = p.D ? p.D[(int64_t)hh * P + p0 + q] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tr + 4 * lq + r;
          if (t < nval) {
            const int64_t gi = (((int64_t)b * L + t0 + t) * H + hh) * P + p0 + q;
            float yv = yd[r] + __builtin_amdgcn_exp2f(sCum[t]) * yo[r] + Dq * bf2f(sU[t * UP + q]);
            if (p.z) yv *= silu_s(bf2f(sZ[t * UP + q]));
            gY[gi] = f2bf(yv);
          }
        }
      }
    }
    // ================= phase 2b: the chunk's state contribution, then the new state ======
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w * SPW + i, tn = k / PT, tp = k % PT;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < Q; kk += 32) {
        const bf16x8 a = ld8(&sBt[(16 * tn + l16) * QP + kk + 8 * lq]);
        const bf16x8 bb = ld8(&sXWt[(16 * tp + l16) * QP + kk + 8 * lq]);
        const bf16x8 bl = ld8(&sXWtl[(16 * tp + l16) * QP + kk + 8 * lq]);
        sacc = mfma(a, bb, sacc);
        sacc = mfma(a, bl, sacc);
      }
      const float dec = __builtin_amdgcn_exp2f(cum_end);
#pragma unroll
      for (int r = 0; r < 4; ++r) hs[i][r] = fmaf(dec, hs[i][r], sacc[r]);
    }
    __syncthreads();       // every wave is done with this chunk's buffers and the old state copy
    store_state_operand();
  }
  // ---- final state
  if (p.h_last) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int k = w * SPW + i, tn = k / PT, tp = k % PT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 16 * tn + 4 * lq + r, q = 16 * tp + l16;
        p.h_last[((int64_t)b * p.dim + (int64_t)hh * P + p0 + q) * N + n] = hs[i][r];
      }
    }
  }
}

template <int N, int PS>
int launch_ps(const KParams& kp, int zoh, hipStream_t st) {
  const dim3 grid(kp.P / PS, kp.H, kp.batch);
  if (zoh) hipLaunchKernelGGL((ssd_kernel<N, PS, true>), grid, dim3(256), 0, st, kp);
  else hipLaunchKernelGGL((ssd_kernel<N, PS, false>), grid, dim3(256), 0, st, kp);
  return (int)hipGetLastError();
}

template <int N>
int launch_n(const KParams& kp, int ps, int zoh, hipStream_t st) {
  switch (ps) {
    case 64: return launch_ps<N, 64>(kp, zoh, st);
    case 32: return launch_ps<N, 32>(kp, zoh, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

// N in {32, 64, 128}; ps (positions per workgroup) in {32, 64} and divides P.
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
