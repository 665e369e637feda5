// valu_rates.hip -- issue-rate measurements of the gfx950 units the scan is bound by.
//
// The rooflines of the per-channel scan need three machine figures that vendor tables do
// not give directly: how many fp32 lanes a SIMD retires per clock without packed math (the
// scan compiles with packed fp32 disabled), what a transcendental (v_exp_f32, v_log_f32,
// v_rcp_f32) costs relative to that, and the shader clock under load.  Each kernel below
// runs 8 independent dependency chains per lane, ITERS x 32 instructions of one kind, on
// a grid of 256 * W workgroups of 4 waves (W waves per SIMD); each wave records its shader
// clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) around the loop.
// The host turns wall time into instructions per second per SIMD and the per-wave counter
// ratio into the clock.  Two HBM kernels (read-only sum, copy) give the streaming rates.
// Built into libssm_rates.so (not the scan library); bench.py --valu-rates runs it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

namespace {

constexpr int ITERS = 4096;

struct WaveRec {
  long long t0, t1, r0, r1;
};

enum Kind { FMA = 0, MUL = 1, EXP2 = 2, LOG2 = 3, RCP = 4, ELEMENT = 5, MIX4 = 6 };

template <int KIND>
__global__ void __launch_bounds__(256) rate_kernel(float* out, WaveRec* rec, float a, float b) {
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  float x[8], e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = threadIdx.x * 1e-3f + i;
    e[i] = -1e-3f * i - threadIdx.x * 1e-6f;
  }
  // scan element operands: step, dt*u and C of the step, B per chain (state), e[] as A
  float dt = 0.01f + threadIdx.x * 1e-6f, du = 0.3f, Cv = 0.25f, acc = 0.0f, Bs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) Bs[i] = 0.5f + 0.01f * i;
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (KIND == ELEMENT) {
        // one element of the per-channel scan per chain: y = dt*A, a = exp2(y), bx = du*B,
        // h = a*h + bx, acc = C*h + acc  (5 instructions, one of them transcendental)
        float accl = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float av = __builtin_amdgcn_exp2f(dt * e[i]);
          x[i] = fmaf(av, x[i], du * Bs[i]);
          accl = fmaf(Cv, x[i], accl);
        }
        acc += accl;
        dt = dt * a + b * 1e-9f;
        du = du * a;
        Cv = Cv * a;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (KIND == FMA) x[i] = fmaf(x[i], a, b);
          if (KIND == MUL) x[i] = x[i] * a;
          if (KIND == EXP2) x[i] = __builtin_amdgcn_exp2f(x[i]);
          if (KIND == LOG2) x[i] = __builtin_amdgcn_logf(x[i]);
          if (KIND == RCP) x[i] = __builtin_amdgcn_rcpf(x[i]);
          if (KIND == MIX4) {   // 4 fma + 1 exp per chain: additive or overlapped?
            e[i] = __builtin_amdgcn_exp2f(e[i]);
            x[i] = fmaf(x[i], a, b);
            x[i] = fmaf(x[i], a, b);
            x[i] = fmaf(x[i], a, b);
            x[i] = fmaf(x[i], a, b);
          }
        }
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = acc;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + e[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) rec[wave] = WaveRec{t0, t1, r0, r1};
}

__global__ void __launch_bounds__(256) hbm_read_kernel(const float4* __restrict__ src, size_t n, float* out) {
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const float4 v = src[i];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (acc.x == 1234.5f) out[0] = acc.y + acc.z + acc.w;   // keeps the loads; never true for zeros
}

__global__ void __launch_bounds__(256) hbm_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                       size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

typedef void (*RateKernel)(float*, WaveRec*, float, float);

RateKernel kernel_of(int kind) {
  switch (kind) {
    case FMA: return rate_kernel<FMA>;
    case MUL: return rate_kernel<MUL>;
    case EXP2: return rate_kernel<EXP2>;
    case LOG2: return rate_kernel<LOG2>;
    case RCP: return rate_kernel<RCP>;
    case ELEMENT: return rate_kernel<ELEMENT>;
    case MIX4: return rate_kernel<MIX4>;
    default: return nullptr;
  }
}

}  // namespace

extern "C" {

// Runs kernel `kind` (0 fma, 1 mul, 2 exp2, 3 log2, 4 rcp, 5 scan element, 6 four fma + one
// exp) with `waves` waves per SIMD on 256 CUs.  res[0] = wall ms (HIP events), res[1] = mean
// shader clock in GHz over the waves, res[2] = instruction units per second per SIMD
// (a unit = one instruction of the kind, or one element / one 4fma+exp group), res[3] =
// shader cycles per unit per SIMD.  Returns 0 or a hipError_t value.
int ssm_rates_run(int kind, int waves, double* res) {
  RateKernel k = kernel_of(kind);
  if (!k || waves < 1 || waves > 8 || !res) return (int)hipErrorInvalidValue;
  const int blocks = 256 * waves;
  float* out = nullptr;
  WaveRec* rec = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)blocks * 256 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&rec, (size_t)blocks * 4 * sizeof(WaveRec));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  float ms = 0.0f;
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, out, rec, 0.999f, 0.001f);   // warm-up
    e = hipDeviceSynchronize();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, 0);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, 0, out, rec, 0.999f, 0.001f);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, 0);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  double clk = 0.0;
  if (e == hipSuccess) {
    WaveRec* h = new WaveRec[(size_t)blocks * 4];
    e = hipMemcpy(h, rec, (size_t)blocks * 4 * sizeof(WaveRec), hipMemcpyDeviceToHost);
    for (int i = 0; e == hipSuccess && i < blocks * 4; ++i)
      clk += (double)(h[i].t1 - h[i].t0) / ((double)(h[i].r1 - h[i].r0) / 100e6);
    delete[] h;
    clk /= (double)blocks * 4;
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (out) hipFree(out);
  if (rec) hipFree(rec);
  if (e != hipSuccess) return (int)e;
  const double units = (double)ITERS * 32 * waves;   // per SIMD
  res[0] = ms;
  res[1] = clk / 1e9;
  res[2] = units / (ms * 1e-3);
  res[3] = clk / res[2];
  return 0;
}

// HBM: res[0] = read-only GB/s, res[1] = copy GB/s (bytes read + written), over `mib` MiB
// buffers, best of 5 launches each for a grid of 4096 workgroups.
int ssm_rates_hbm(int mib, double* res) {
  if (mib < 1 || !res) return (int)hipErrorInvalidValue;
  const size_t bytes = (size_t)mib << 20;
  float4 *a = nullptr, *b = nullptr;
  float* out = nullptr;
  hipError_t e = hipMalloc(&a, bytes);
  if (e == hipSuccess) e = hipMalloc(&b, bytes);
  if (e == hipSuccess) e = hipMalloc(&out, 16);
  if (e == hipSuccess) e = hipMemset(a, 0, bytes);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  const size_t n = bytes / 16;
  double best_r = 0.0, best_c = 0.0;
  for (int rep = 0; e == hipSuccess && rep < 6; ++rep) {
    float ms = 0.0f;
    e = hipEventRecord(e0, 0);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(hbm_read_kernel, dim3(4096), dim3(256), 0, 0, a, n, out);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && rep > 0) best_r = std::max(best_r, bytes / (ms * 1e-3) / 1e9);
    if (e == hipSuccess) e = hipEventRecord(e0, 0);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(hbm_copy_kernel, dim3(4096), dim3(256), 0, 0, a, b, n);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, 0);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && rep > 0) best_c = std::max(best_c, 2.0 * bytes / (ms * 1e-3) / 1e9);
  }
  if (e0) hipEventDestroy(e0);
  if (e1) hipEventDestroy(e1);
  if (a) hipFree(a);
  if (b) hipFree(b);
  if (out) hipFree(out);
  if (e != hipSuccess) return (int)e;
  res[0] = best_r;
  res[1] = best_c;
  return 0;
}

}  // extern "C"
