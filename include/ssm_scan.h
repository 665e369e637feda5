/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan (S6).
 *
 * The operation («Mamba 选择性状态空间模型：亚二次复杂度大语言模型推理工程实践» §2.2, §3.2,
 * §4.1-§4.2; «Mamba与SSM状态空间模型：一张摘要卡读完万页档案», sections 离散化变换 and
 * 选择性机制; «AI底层架构的一场革命：Mamba如何用「状态压缩」挑战Transformer的十年统治»,
 * section "Mamba Block：完整模块结构"):
 *
 *   for every (batch b, channel d, state n), over t = 0 .. L-1:
 *     dt_t  = softplus(delta_t + delta_bias)      (or delta_t + delta_bias if softplus_flag == 0)
 *     h_t   = exp(dt_t * A) * h_{t-1} + dt_t * B_t * u_t          h_{-1} = h0 (or 0)
 *             (with dims->discretization == SSM_DISC_ZOH the input term is the exact
 *              zero-order hold expm1(dt_t * A) / A * B_t * u_t of «Mamba 选择性状态空间模型» §2.2)
 *     y_t   = (sum_n C_t[n] * h_t[n] + D * u_t) * SiLU(z_t)       (D, z optional)
 *   and h_last = h_{L-1}.
 *
 * Everything is computed in float32 with float32 state; u, delta, B, C, z and
 * y are stored in io_dtype (float32 or bfloat16), A, D, delta_bias, h0 and
 * h_last are float32.
 *
 * Layouts (all tensors contiguous, innermost index last):
 *   SSM_LAYOUT_BDL  (per-channel state, one A per (channel, state)):
 *       u, delta, z, y : (batch, dim, seqlen)
 *       B, C           : (batch, ngroups, dstate, seqlen)   channel d uses group d / (dim/ngroups)
 *       A              : (dim, dstate)
 *       delta_bias, D  : (dim)
 *   SSM_LAYOUT_BLHP (multi-head state, one scalar A per head; dim = nheads*headdim):
 *       u, z, y        : (batch, seqlen, nheads, headdim)
 *       delta          : (batch, seqlen, nheads)
 *       B, C           : (batch, seqlen, ngroups, dstate)   head h uses group h / (nheads/ngroups)
 *       A, delta_bias  : (nheads)
 *       D              : (dim)                               channel d = h*headdim + p
 *   h0, h_last         : (batch, dim, dstate) float32 in both layouts.
 *
 * Ownership: every pointer is a device pointer owned by the caller; the
 * library keeps none of them after the call returns.  Outputs y and h_last
 * must not overlap any input or each other.  All tensor base pointers must be
 * 16-byte aligned.
 *
 * Execution: ssm_scan_fwd validates its arguments on the host before any HIP
 * call, then enqueues its kernels on `stream` (a hipStream_t; NULL is the
 * default stream) and returns without synchronising.  Faults inside a kernel
 * surface at the caller's next synchronisation on that stream.  The call is
 * reentrant; calls on different streams may overlap when each has its own
 * workspace.
 *
 * Workspace: long sequences are split into time segments whose carries are
 * combined by the library (the chunked scan of «Mamba 选择性状态空间模型» §4.1 and
 * the state continuation of §7.2).  The scratch they need is
 * ssm_scan_workspace_size(dims) bytes.  If dims->workspace is NULL and the size is
 * nonzero, the library allocates it stream-ordered (hipMallocAsync /
 * hipFreeAsync on `stream`); otherwise dims->workspace must hold at least
 * that many bytes (SSM_ERR_WORKSPACE if dims->workspace_bytes is smaller).
 * With a caller workspace (or a zero size) a call enqueues kernel launches
 * only (no allocation, no memset, no copy), so it may be captured in a HIP
 * graph; the graph then reads and writes the same addresses on every replay.
 *
 * Errors: every entry point returns SSM_OK (0) or a negative code; no C++
 * exception crosses the ABI.  ssm_strerror(code) gives a static message; for
 * SSM_ERR_HIP it also carries the HIP error text of the failing call (kept
 * per thread until that thread's next ssm_scan_fwd).
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_LAYOUT_BDL 0
#define SSM_LAYOUT_BLHP 1

#define SSM_F32 0
#define SSM_BF16 1

/* ssm_dims_t.discretization: how B̄ is formed from the step size */
#define SSM_DISC_DELTA_B 0 /* B̄ = Δ·B (default; zero-initialised dims select it) */
#define SSM_DISC_ZOH 1     /* exact zero-order hold: B̄ = (ΔA)^-1 (exp(ΔA) - 1) Δ·B = expm1(ΔA)/A · B */

#define SSM_OK 0
#define SSM_ERR_NULL_ARG -1    /* u, delta, A, B, C, y or dims is NULL */
#define SSM_ERR_BAD_DIMS -2    /* a size <= 0, nheads*headdim != dim, groups do not divide, ... */
#define SSM_ERR_UNSUPPORTED -3 /* unknown layout, io_dtype or discretization; dstate outside 1..256 */
#define SSM_ERR_ALIGN -4       /* a tensor pointer is not 16-byte aligned */
#define SSM_ERR_ALIAS -5       /* y or h_last overlaps an input or each other */
#define SSM_ERR_WORKSPACE -6   /* caller workspace smaller than ssm_scan_workspace_size */
#define SSM_ERR_HIP -7         /* a HIP runtime call failed (see ssm_strerror) */
#define SSM_ERR_SCRATCH -8     /* ssm_scan_fwd_noalloc: the launch needs more than the static scratch */

typedef struct ssm_dims {
  int64_t batch;     /* B >= 1 */
  int64_t seqlen;    /* L >= 1 */
  int64_t dim;       /* D = channels (= nheads*headdim for BLHP) */
  int64_t dstate;    /* N, 1..256 */
  int64_t nheads;    /* BLHP: H >= 1; BDL: ignored */
  int64_t headdim;   /* BLHP: P >= 1; BDL: ignored */
  int64_t ngroups;   /* G >= 1; divides dim (BDL) or nheads (BLHP) */
  int32_t layout;    /* SSM_LAYOUT_BDL or SSM_LAYOUT_BLHP */
  int32_t io_dtype;  /* SSM_F32 or SSM_BF16 */
  void* workspace;          /* optional device scratch, see above */
  size_t workspace_bytes;   /* its size in bytes */
  int32_t discretization;   /* SSM_DISC_DELTA_B (0) or SSM_DISC_ZOH (1); other values: SSM_ERR_UNSUPPORTED */
  int32_t reserved;         /* must be 0 */
} ssm_dims_t;

/*
 * Selective scan forward.  A, B, C, u, delta, y are required; D, z,
 * delta_bias, h0 and h_last may be NULL (no skip term, no gate, zero bias,
 * zero initial state, final state not wanted).  softplus_flag != 0 applies
 * softplus to delta + delta_bias.  `stream` is a hipStream_t (may be NULL).
 */
int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus_flag,
                 const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream);

/*
 * Single-token state update (decode): one step of the same recurrence, the
 * constant-time, constant-memory per-token update of generation
 * («Mamba与SSM状态空间模型：一张摘要卡读完万页档案», section 线性扫描算法;
 * «Mamba 选择性状态空间模型：亚二次复杂度大语言模型推理工程实践» §6.2).  It equals
 * ssm_scan_fwd with seqlen = 1: dims->seqlen must be 1 (else SSM_ERR_BAD_DIMS),
 * and the tensors have the scan layouts with the time axis of length 1:
 *   SSM_LAYOUT_BDL : x, z, y, delta (batch, dim); B, C (batch, ngroups, dstate);
 *                    A (dim, dstate); delta_bias, D (dim)
 *   SSM_LAYOUT_BLHP: x, z, y (batch, nheads, headdim); delta (batch, nheads);
 *                    B, C (batch, ngroups, dstate); A, delta_bias (nheads); D (dim)
 *   h_in, h_out    : (batch, dim, dstate) float32.
 * h_in NULL means a zero state; h_out NULL means the new state is not stored.
 * h_out may be the same pointer as h_in (update in place) but must not overlap
 * any other input or y.  Needs no workspace.  Errors as for ssm_scan_fwd.
 */
int ssm_state_update(const void* x, const void* delta, const float* A, const void* B, const void* C,
                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                     const float* h_in, float* h_out, void* y, const ssm_dims_t* dims, void* stream);

/*
 * Input stage of the Mamba block fused into the scan: the raw input x passes
 * through a causal depthwise 1-D convolution and SiLU, and the result is the u
 * of the recurrence (in dt*u and in the D*u skip).  («AI底层架构的一场革命：Mamba如何用
 * 「状态压缩」挑战Transformer的十年统治», section "Mamba Block：完整模块结构": x_proj ->
 * 1-D convolution -> SiLU -> S6; «Mamba与SSM状态空间模型：一张摘要卡读完万页档案»,
 * section "Mamba架构设计".)  The pages give no width: width is 1..4, and
 *   u_t = SiLU(bias[d] + sum_{j<width} weight[d][j] * x_{t-width+1+j})
 * where inputs before t = 0 come from state_in (or are 0).
 */
typedef struct ssm_conv {
  const float* weight;  /* (dim, width) float32, required */
  const float* bias;    /* (dim) float32, or NULL */
  const float* state_in;/* (batch, dim, width-1) float32: the raw inputs before t = 0, oldest first; or NULL */
  float* state_out;     /* (batch, dim, width-1) float32: the last width-1 raw inputs; or NULL */
  int32_t width;        /* 1..4 */
  int32_t reserved;     /* must be 0 */
} ssm_conv_t;

/*
 * ssm_scan_fwd with the input stage above; x has the layout and dtype of u, and
 * channel d of weight, bias and the states is h*headdim + p in SSM_LAYOUT_BLHP.
 * Supported for SSM_LAYOUT_BDL with dstate <= 32 and seqlen <= 2^26 (the
 * per-channel kernels) and for SSM_LAYOUT_BLHP with bfloat16 storage, dstate in
 * {32, 64, 128} and headdim a multiple of 16 (the chunked kernel); other shapes
 * return SSM_ERR_UNSUPPORTED.  conv or conv->weight NULL:
 * SSM_ERR_NULL_ARG; width outside 1..4: SSM_ERR_UNSUPPORTED.  state_out must
 * not overlap any input or output.  Workspace, stream and errors as for
 * ssm_scan_fwd (ssm_scan_workspace_size gives the scratch size).
 */
int ssm_conv_scan_fwd(const void* x, const ssm_conv_t* conv, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias, int softplus_flag,
                      const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream);

/*
 * Allocation-free variant of ssm_scan_fwd, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, layouts, validation, stream semantics and errors are those of ssm_scan_fwd,
 * except that dims->workspace and dims->workspace_bytes are ignored: the scratch comes from
 * a static device array of ssm_scan_scratch_capacity() bytes (32 MiB) that the library holds
 * on every GPU it runs on until the process ends.  The call makes no hipMalloc/hipFree, no
 * stream-ordered allocation and no other allocating call.  A launch that needs more scratch
 * than the array holds (ssm_scan_workspace_size(dims) > ssm_scan_scratch_capacity()) returns
 * SSM_ERR_SCRATCH before any HIP call.  On its first call on a device (with that device
 * current) it looks the array's device address up; a failure there returns SSM_ERR_HIP.
 * All calls on one GPU share that GPU's array, so calls that overlap in time on one GPU
 * (other streams, other host threads) race on it and must be serialised by the caller.
 */
int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int softplus_flag,
                         const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream);

/* Bytes of the static device scratch ssm_scan_fwd_noalloc uses (per GPU). */
size_t ssm_scan_scratch_capacity(void);

/* Bytes of scratch ssm_scan_fwd needs for these dims (0 if none); 0 also for invalid dims. */
size_t ssm_scan_workspace_size(const ssm_dims_t* dims);

/* Static description of an error code (never NULL). */
const char* ssm_strerror(int code);

/*
 * Writes a one-line description of the launch plan chosen for dims
 * (kernel variant, grid, time segments) into buf; returns SSM_OK or an
 * error code for invalid dims.  Makes no HIP call.
 */
int ssm_scan_describe(const ssm_dims_t* dims, char* buf, size_t buf_len);

/* Library ABI version (major*10000 + minor*100 + patch). */
int ssm_scan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
