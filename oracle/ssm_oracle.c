/*
 * ssm_oracle.c -- fp64 CPU oracle for the selective state-space scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg use it.  It shares no source with the HIP library.
 *
 * What it computes is the plain sequential recurrence, written out in the
 * order and notation of the pages, in double precision:
 *
 *   Delta_t = softplus(Delta_raw_t + bias)          «Mamba 选择性状态空间模型：亚二次复杂度
 *                                                    大语言模型推理工程实践» §3.2 (Δ_t as the
 *                                                    softplus of a projection plus a broadcast
 *                                                    bias); softplus = log(1+e^z) per
 *                                                    «Mamba与SSM状态空间模型：一张摘要卡读完万页档案»,
 *                                                    section "Python 演示"
 *   Abar_t  = exp(Delta_t * A)                      «Mamba与SSM状态空间模型» section "离散化变换"
 *                                                    and "选择性机制" (e^{Δ_t A}); same page-1 §2.2
 *   Bbar_t x_t = Delta_t * B_t * x_t                «Mamba与SSM状态空间模型» "离散化变换" (B̄ = Δ B)
 *     or, with discretization = 1, the exact zero-order hold of
 *   Bbar_t = (Delta_t A)^-1 (exp(Delta_t A) - 1) Delta_t B_t   «Mamba 选择性状态空间模型» §2.2
 *            = expm1(Delta_t A) / A * B_t  (Delta_t B_t when A = 0)
 *   h_t     = Abar_t * h_{t-1} + Bbar_t x_t         «Mamba 选择性状态空间模型» §2.2 and §4.1
 *   y_t     = C_t . h_t + D * x_t                   «Mamba 选择性状态空间模型» §2.2 (output eq.);
 *                                                    «Transformer架构遭遇颠覆性突破» §二.1
 *   y_t    *= SiLU(z_t)   (optional gate)           «AI底层架构的一场革命：Mamba如何用「状态压缩」
 *                                                    挑战Transformer的十年统治», section
 *                                                    "Mamba Block：完整模块结构" (y_ssm ⊙ SiLU(z))
 *   h_L is returned as the final state               «Mamba 选择性状态空间模型» §4.2 (only the
 *                                                    final state is written back) and §7.2
 *                                                    (state continuation across chunks)
 *
 * A is real and diagonal: one value per (channel, state) in the (B,D,L)
 * layout, one scalar per head in the (B,L,H,P) multi-head layout
 * («AI底层架构的一场革命» section "Mamba-2：状态空间对偶性理论" names the
 * multi-head SSM).  The readout sums over the state index, as in the
 * page «State Space Models 深度实战：从 S4 到 Mamba 的架构演进与 CUDA 优化» §5.2.
 *
 * Readings where the pages are silent:
 *  - softplus is evaluated in the overflow-free form max(r,0)+log1p(exp(-|r|)),
 *    which equals log(1+e^r) exactly in real arithmetic;
 *  - SiLU(z) = z / (1 + e^{-z});
 *  - the gate multiplies the whole S6 output including the D*x skip;
 *  - D, z, bias and h0 are optional (NULL means 0 / no gate / zero state);
 *  - the optional input stage (oracle_conv_scan_f64) is the Mamba block's 1-D
 *    convolution then SiLU in front of the SSM («AI底层架构的一场革命», section
 *    "Mamba Block：完整模块结构"; «Mamba与SSM状态空间模型», section "Mamba架构设计");
 *    the pages give neither width nor padding: it is read as causal (step t sees
 *    inputs t-K+1..t), depthwise (one filter of width K per channel, plus a bias),
 *    with the K-1 inputs before t = 0 taken from a carried state (zeros if none);
 *  - the zero-order-hold B̄ as printed on page 1 §2.2 lacks the factor Δ on B;
 *    it is read as the exact hold of a constant input over one step, whose
 *    first-order form is the Δ·B of the other pages.
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t batch, seqlen, dim, dstate, nheads, headdim, ngroups;
  int32_t layout;   /* 0: (B,D,L) Mamba-1 layout; 1: (B,L,H,P) multi-head layout */
  int32_t io_dtype; /* 0: float32 storage; 1: bfloat16 storage (raw uint16 bits) */
  int32_t discretization; /* 0: Bbar = Delta*B; 1: exact zero-order hold */
  int32_t reserved;
} oracle_dims;

/* bfloat16 bits -> double: a bfloat16 is the upper half of a float32. */
static double bf16_bits_to_double(uint16_t bits) {
  uint32_t w = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static double load_io(const void* p, int64_t i, int32_t io_dtype) {
  if (io_dtype == 1) return bf16_bits_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

double oracle_softplus(double r) {
  /* log(1 + e^r), overflow-free form (identical in real arithmetic) */
  return (r > 0.0 ? r : 0.0) + log1p(exp(-fabs(r)));
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct {
  const void *u, *delta, *B, *C, *z;
  const float *A, *D, *bias, *h0;
  int softplus;
  const float *conv_w, *conv_b, *conv_state_in; /* optional causal depthwise conv + SiLU stage */
  int conv_k;
  double* conv_state_out;
  oracle_dims dims;
  const int64_t* t_out; /* sorted list of time indices whose y is emitted; NULL: all */
  int64_t n_t_out;
  double* y;
  double* h_last;
  int64_t row_begin, row_end; /* rows are (b, d) pairs, d = h*P + p in the multi-head layout */
} job_t;

static void scan_rows(const job_t* J) {
  const oracle_dims* m = &J->dims;
  const int64_t Bsz = m->batch, L = m->seqlen, Dm = m->dim, N = m->dstate;
  const int64_t G = m->ngroups;
  const int64_t H = (m->layout == 1) ? m->nheads : Dm;
  const int64_t P = (m->layout == 1) ? m->headdim : 1;
  double* h = (double*)malloc(sizeof(double) * (size_t)N);
  const int K = J->conv_k;                    /* 0: no input stage */
  double win[16];                             /* the K-1 previous raw inputs, oldest first */
  (void)Bsz;
  for (int64_t row = J->row_begin; row < J->row_end; ++row) {
    const int64_t b = row / Dm, d = row % Dm;
    const int64_t hd = d / P, p = d % P;       /* head and position within head */
    const int64_t g = hd / (H / G);            /* group of this head / channel */
    for (int64_t n = 0; n < N; ++n) h[n] = J->h0 ? (double)J->h0[row * N + n] : 0.0;
    for (int k = 0; k + 1 < K; ++k) win[k] = J->conv_state_in ? (double)J->conv_state_in[row * (K - 1) + k] : 0.0;
    int64_t k_out = 0;
    for (int64_t t = 0; t < L; ++t) {
      int64_t i_x, i_dt, i_bc;
      if (m->layout == 0) {
        i_x = row * L + t;                      /* u, z, y, delta: (B, D, L) */
        i_dt = i_x;
        i_bc = (b * G + g) * N * L + t;         /* B, C: (B, G, N, L); + n*L */
      } else {
        i_x = ((b * L + t) * H + hd) * P + p;   /* u, z, y: (B, L, H, P) */
        i_dt = (b * L + t) * H + hd;            /* delta: (B, L, H) */
        i_bc = ((b * L + t) * G + g) * N;       /* B, C: (B, L, G, N); + n */
      }
      const int64_t bc_stride = (m->layout == 0) ? L : 1;
      const double bias = J->bias ? (double)J->bias[m->layout == 0 ? d : hd] : 0.0;
      const double r = load_io(J->delta, i_dt, m->io_dtype) + bias;
      const double dt = J->softplus ? oracle_softplus(r) : r;
      double x = load_io(J->u, i_x, m->io_dtype);
      if (K > 0) {
        /* causal depthwise convolution over the raw inputs t-K+1..t, then SiLU */
        double c = J->conv_b ? (double)J->conv_b[d] : 0.0;
        for (int k = 0; k + 1 < K; ++k) c += (double)J->conv_w[d * K + k] * win[k];
        c += (double)J->conv_w[d * K + K - 1] * x;
        for (int k = 0; k + 2 < K; ++k) win[k] = win[k + 1];
        if (K > 1) win[K - 2] = x;
        x = oracle_silu(c);
      }
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double A = (m->layout == 0) ? (double)J->A[d * N + n] : (double)J->A[hd];
        const double Bn = load_io(J->B, i_bc + n * bc_stride, m->io_dtype);
        const double Cn = load_io(J->C, i_bc + n * bc_stride, m->io_dtype);
        const double abar = exp(dt * A);
        /* Bbar / B: Delta, or expm1(Delta A) / A for the exact hold (Delta when A = 0) */
        const double bbar = (m->discretization == 1 && A != 0.0) ? expm1(dt * A) / A : dt;
        h[n] = abar * h[n] + bbar * Bn * x;
        acc += Cn * h[n];
      }
      double yt = acc + (J->D ? (double)J->D[d] : 0.0) * x;
      if (J->z) yt *= oracle_silu(load_io(J->z, i_x, m->io_dtype));
      /* emit y_t if t is selected */
      if (J->t_out == NULL) {
        if (m->layout == 0) J->y[row * L + t] = yt;
        else J->y[((b * L + t) * H + hd) * P + p] = yt;
      } else if (k_out < J->n_t_out && J->t_out[k_out] == t) {
        const int64_t T = J->n_t_out;
        if (m->layout == 0) J->y[row * T + k_out] = yt;
        else J->y[((b * T + k_out) * H + hd) * P + p] = yt;
        ++k_out;
      }
    }
    if (J->h_last)
      for (int64_t n = 0; n < N; ++n) J->h_last[row * N + n] = h[n];
    if (J->conv_state_out)
      for (int k = 0; k + 1 < K; ++k) J->conv_state_out[row * (K - 1) + k] = win[k];
  }
  free(h);
}

static void* scan_thread(void* arg) {
  scan_rows((const job_t*)arg);
  return NULL;
}

/*
 * Returns 0 on success, -1 on bad arguments.  All pointers are host pointers.
 * y has the layout of u with the time axis restricted to t_out (if given;
 * t_out must be strictly increasing).  h_last is (B, D, N) in float64.
 */
int oracle_conv_scan_f64(const void* u, const float* conv_w, const float* conv_b, int conv_k,
                         const float* conv_state_in, double* conv_state_out, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                         int softplus, const float* h0, const oracle_dims* dims, const int64_t* t_out,
                         int64_t n_t_out, double* y, double* h_last, int nthreads);

int oracle_scan_f64(const void* u, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const void* z, const float* delta_bias, int softplus,
                    const float* h0, const oracle_dims* dims, const int64_t* t_out, int64_t n_t_out,
                    double* y, double* h_last, int nthreads) {
  return oracle_conv_scan_f64(u, NULL, NULL, 0, NULL, NULL, delta, A, B, C, D, z, delta_bias, softplus, h0, dims,
                              t_out, n_t_out, y, h_last, nthreads);
}

/*
 * Same scan with the raw input u first passed through the causal depthwise
 * convolution (weights (D, conv_k) float32, bias (D) or NULL) and SiLU; the
 * conv_k - 1 inputs before t = 0 come from conv_state_in (B, D, conv_k-1) or
 * are 0, and conv_state_out (B, D, conv_k-1) receives the last conv_k - 1 raw
 * inputs.  Both layouts: the convolution runs along time per channel d (d = h*P + p
 * in the multi-head layout, whose x is read at (b, t, h, p)); conv_k in 1..16.
 */
int oracle_conv_scan_f64(const void* u, const float* conv_w, const float* conv_b, int conv_k,
                         const float* conv_state_in, double* conv_state_out, const void* delta, const float* A,
                         const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                         int softplus, const float* h0, const oracle_dims* dims, const int64_t* t_out,
                         int64_t n_t_out, double* y, double* h_last, int nthreads) {
  if (!u || !delta || !A || !B || !C || !dims || !y) return -1;
  if (conv_k < 0 || conv_k > 16 || (conv_k > 0 && !conv_w)) return -1;
  const oracle_dims m = *dims;
  if (m.batch <= 0 || m.seqlen <= 0 || m.dim <= 0 || m.dstate <= 0 || m.ngroups <= 0) return -1;
  if (m.discretization != 0 && m.discretization != 1) return -1;
  if (m.layout == 1) {
    if (m.nheads <= 0 || m.headdim <= 0 || m.nheads * m.headdim != m.dim) return -1;
    if (m.nheads % m.ngroups) return -1;
  } else if (m.layout == 0) {
    if (m.dim % m.ngroups) return -1;
  } else {
    return -1;
  }
  if (t_out) {
    for (int64_t k = 0; k < n_t_out; ++k) {
      if (t_out[k] < 0 || t_out[k] >= m.seqlen) return -1;
      if (k > 0 && t_out[k] <= t_out[k - 1]) return -1;
    }
  }
  const int64_t rows = m.batch * m.dim;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int i = 0; i < nthreads; ++i) {
    job_t* J = &jobs[i];
    J->u = u; J->delta = delta; J->B = B; J->C = C; J->z = z;
    J->A = A; J->D = D; J->bias = delta_bias; J->h0 = h0; J->softplus = softplus;
    J->conv_w = conv_w; J->conv_b = conv_b; J->conv_k = conv_k;
    J->conv_state_in = conv_state_in; J->conv_state_out = conv_state_out;
    J->dims = m; J->t_out = t_out; J->n_t_out = n_t_out; J->y = y; J->h_last = h_last;
    J->row_begin = rows * i / nthreads;
    J->row_end = rows * (i + 1) / nthreads;
  }
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, scan_thread, &jobs[i]);
  scan_rows(&jobs[0]);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(jobs);
  free(th);
  return 0;
}
