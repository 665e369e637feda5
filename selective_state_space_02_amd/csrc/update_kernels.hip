// update_kernels.hip -- gfx950 kernel of the single-token state update (decode).
//
// Generating one token advances every layer's state by exactly one step of the
// recurrence, in constant time and memory (the O(1) per-token update of
// «Mamba与SSM状态空间模型：一张摘要卡读完万页档案», section 线性扫描算法; the
// incremental one-step update of «Mamba 选择性状态空间模型：亚二次复杂度大语言模型推理工程实践»
// §6.2).  Per (batch b, channel d, state n):
//   dt = softplus(delta + bias);  h' = exp(dt A) h + dt x B[n];  y = (sum_n C[n] h' + D x) SiLU(z)
// It is the seqlen = 1 case of the scan and is bound by HBM traffic on the state
// (read once, written once), so the mapping is chosen for coalescing: LPR lanes
// cover one channel's state vector (NS consecutive states per lane), the readout
// sum is a cross-lane butterfly inside those LPR lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_plan.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct F32 {
  static __device__ float ld(const void* p, int64_t i) { return ((const float*)p)[i]; }
  static __device__ void st(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
};
struct BF16 {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  static __device__ float ld(const void* p, int64_t i) {
    return __uint_as_float(((uint32_t)((const uint16_t*)p)[i]) << 16);
  }
  static __device__ void st(void* p, int64_t i, float v) {
    const bf16x2 w = {(__bf16)v, (__bf16)0.0f};
    ((uint16_t*)p)[i] = (uint16_t)(__builtin_bit_cast(uint32_t, w) & 0xffffu);
  }
};

// softplus(r) = max(r, 0) + log1p(e^-|r|), log1p(e) = log(w) + (e - (w - 1)) with w = fl(1 + e)
__device__ __forceinline__ float softplus_u(float r) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(r) * kLog2e);
  const float w = 1.0f + e;
  const float err = e - (w - 1.0f);
  return (r > 0.0f ? r : 0.0f) + fmaf(__builtin_amdgcn_logf(w), kLn2, err);
}

// LAYOUT 0 (B,D): A per (channel, state), delta/bias per channel.
// LAYOUT 1 (B,H,P): A, delta, bias per head.
// LPR lanes per channel, NS consecutive states per lane (VEC: NS = 4 as one 16-byte
// access; otherwise one state per lane).  Each thread takes RPT channels, spaced one
// wave-row-block apart, and issues all of their loads before any arithmetic, so
// every lane keeps RPT independent HBM reads in flight.
template <typename IO, int LAYOUT, int LPR, int NS, bool VEC, int RPT>
__global__ void __launch_bounds__(256) state_update_kernel(UParams p) {
  constexpr int RPW = 64 / LPR;   // channels per wave and row block
  const int lane = threadIdx.x & 63;
  const int k = lane % LPR;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int N = p.N;

  int64_t rr[RPT];
  bool ok[RPT];
  float xv[RPT], raw[RPT], zv[RPT], hv[RPT][NS], Av[RPT][NS], Bv[RPT][NS], Cv[RPT][NS];
  // ---- loads of all RPT channels
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int64_t r = (wave * RPT + i) * RPW + lane / LPR;    // b*dim + d
    ok[i] = r < p.rows;
    rr[i] = ok[i] ? r : 0;
    const int b = (int)(rr[i] / p.dim), d = (int)(rr[i] % p.dim);
    const int head = LAYOUT == 0 ? d : d / p.P;
    const int g = LAYOUT == 0 ? d / p.rows_per_group : head / p.heads_per_group;
    const int64_t di = LAYOUT == 0 ? rr[i] : (int64_t)b * p.H + head;
    raw[i] = IO::ld(p.delta, di) + (p.bias ? p.bias[head] : 0.0f);
    xv[i] = IO::ld(p.x, rr[i]);
    zv[i] = p.z ? IO::ld(p.z, rr[i]) : 0.0f;
    const int64_t bc = ((int64_t)b * p.G + g) * N;
    const int n0 = k * NS;
    if (VEC) {
      const float4 h4 = p.h_in ? *(const float4*)&p.h_in[rr[i] * N + n0] : make_float4(0.f, 0.f, 0.f, 0.f);
      hv[i][0] = h4.x; hv[i][1] = h4.y; hv[i][2] = h4.z; hv[i][3] = h4.w;
      if (LAYOUT == 0) {
        const float4 a4 = *(const float4*)&p.A[(int64_t)d * N + n0];
        Av[i][0] = a4.x; Av[i][1] = a4.y; Av[i][2] = a4.z; Av[i][3] = a4.w;
      } else {
#pragma unroll
        for (int j = 0; j < NS; ++j) Av[i][j] = p.A[head];
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) { Bv[i][j] = IO::ld(p.B, bc + n0 + j); Cv[i][j] = IO::ld(p.C, bc + n0 + j); }
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int n = n0 + j;
        const bool v = n < N;
        const int nc = v ? n : 0;
        hv[i][j] = (p.h_in && v) ? p.h_in[rr[i] * N + nc] : 0.0f;
        Av[i][j] = LAYOUT == 0 ? p.A[(int64_t)d * N + nc] : p.A[head];
        Bv[i][j] = v ? IO::ld(p.B, bc + nc) : 0.0f;
        Cv[i][j] = v ? IO::ld(p.C, bc + nc) : 0.0f;
      }
    }
  }
  // ---- the step, the readout and the stores
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float dt = p.softplus ? softplus_u(raw[i]) : raw[i];
    const float dtx = dt * xv[i];
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float x = dt * Av[i][j];
      const float a = __builtin_amdgcn_exp2f(x * kLog2e);
      float bx = dtx * Bv[i][j];
      if (p.zoh) {   // exact zero-order hold: times expm1(x)/x (Taylor below |x| = 1/8)
        const float poly = fmaf(x, fmaf(x, fmaf(x, fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f), 1.0f);
        bx *= fabsf(x) < 0.125f ? poly : (a - 1.0f) * __builtin_amdgcn_rcpf(x);
      }
      hv[i][j] = fmaf(a, hv[i][j], bx);
      acc = fmaf(Cv[i][j], hv[i][j], acc);
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o /= 2) acc += __shfl_xor(acc, o, LPR);
    if (p.h_out && ok[i]) {
      const int n0 = k * NS;
      if (VEC) {
        *(float4*)&p.h_out[rr[i] * N + n0] = make_float4(hv[i][0], hv[i][1], hv[i][2], hv[i][3]);
      } else {
#pragma unroll
        for (int j = 0; j < NS; ++j)
          if (n0 + j < N) p.h_out[rr[i] * N + n0 + j] = hv[i][j];
      }
    }
    if (k == 0 && ok[i]) {
      const int d = (int)(rr[i] % p.dim);
      float yv = fmaf(p.D ? p.D[d] : 0.0f, xv[i], acc);
      if (p.z) yv *= zv[i] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv[i] * kLog2e));
      IO::st(p.y, rr[i], yv);
    }
  }
}

template <typename IO, int LAYOUT, int LPR, int NS, bool VEC>
int launch_update_v(const UParams& p, hipStream_t st) {
  constexpr int RPT = 2;   // measured: more waves beat more channels per thread at this size
  constexpr int rows_per_block = 4 * (64 / LPR) * RPT;        // 4 waves x channels per wave x RPT
  const int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL((state_update_kernel<IO, LAYOUT, LPR, NS, VEC, RPT>), dim3((unsigned)blocks), dim3(256), 0,
                     st, p);
  return (int)hipGetLastError();
}

template <typename IO, int LAYOUT>
int launch_update_io(const UParams& p, int Npad, hipStream_t st) {
  if (p.N == Npad) {    // unpadded power-of-two state rows: 4 states per lane (16 bytes), N/4 lanes per channel
    switch (Npad) {
      case 16: return launch_update_v<IO, LAYOUT, 4, 4, true>(p, st);
      case 32: return launch_update_v<IO, LAYOUT, 8, 4, true>(p, st);
      case 64: return launch_update_v<IO, LAYOUT, 16, 4, true>(p, st);
      case 128: return launch_update_v<IO, LAYOUT, 32, 4, true>(p, st);
      case 256: return launch_update_v<IO, LAYOUT, 64, 4, true>(p, st);
      default: break;
    }
  }
  switch (Npad) {
    case 16: return launch_update_v<IO, LAYOUT, 16, 1, false>(p, st);
    case 32: return launch_update_v<IO, LAYOUT, 32, 1, false>(p, st);
    case 64: return launch_update_v<IO, LAYOUT, 64, 1, false>(p, st);
    case 128: return launch_update_v<IO, LAYOUT, 64, 2, false>(p, st);
    case 256: return launch_update_v<IO, LAYOUT, 64, 4, false>(p, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_update(const UParams& p, int layout, int io, int Npad, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (layout == SSM_LAYOUT_BDL)
    return io == SSM_BF16 ? launch_update_io<BF16, 0>(p, Npad, st) : launch_update_io<F32, 0>(p, Npad, st);
  return io == SSM_BF16 ? launch_update_io<BF16, 1>(p, Npad, st) : launch_update_io<F32, 1>(p, Npad, st);
}

}  // namespace ssm
