// scan_api.cpp -- C ABI of the selective scan: argument validation, launch plan,
// workspace, error reporting.  Declared in include/ssm_scan.h.
//
// Validation runs entirely on the host and makes no HIP call, so every error
// path can be exercised without a GPU.  The plan splits time into segments only
// when the rows alone cannot fill the chip (the chunked scan with carries of
// «Mamba 选择性状态空间模型：亚二次复杂度大语言模型推理工程实践» §4.1 and the state
// continuation of §7.2).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "scan_plan.h"
#include "ssm_scan.h"

namespace ssm {

namespace {

constexpr int kCUs = 256;   // MI355X compute units

thread_local char g_hip_msg[256] = {0};

int64_t round_up(int64_t x, int64_t m) { return ((x + m - 1) / m) * m; }

// Segment count: enough parallel units (waves for the row-group kernel, workgroups
// otherwise) to fill the chip, but no segment shorter than kMinSeg steps.
// SSM_SCAN_SEGMENTS=<n> overrides (tests, tuning).
int choose_segments(int64_t L, int64_t units, int64_t target, int TB, int64_t* seg_len) {
  constexpr int64_t kMinSeg = 256;
  int64_t nseg = 1;
  const char* env = std::getenv("SSM_SCAN_SEGMENTS");
  if (env && *env) {
    nseg = std::atoi(env);
    if (nseg < 1) nseg = 1;
  } else if (units < target / 2) {
    nseg = (target + units - 1) / units;
    const int64_t max_seg = (L + kMinSeg - 1) / kMinSeg;
    if (nseg > max_seg) nseg = max_seg;
    if (nseg < 1) nseg = 1;
  }
  int64_t len = (L + nseg - 1) / nseg;
  len = round_up(len, TB);
  if (len < TB) len = TB;
  nseg = (L + len - 1) / len;
  if (nseg > 65535) {  // grid z limit: grow the segments instead
    len = round_up((L + 65534) / 65535, TB);
    nseg = (L + len - 1) / len;
  }
  *seg_len = len;
  return (int)nseg;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x0 = (uintptr_t)a, x1 = x0 + na, y0 = (uintptr_t)b, y1 = y0 + nb;
  return x0 < y1 && y0 < x1;
}

bool misaligned(const void* p) { return p && ((uintptr_t)p & 15u); }

}  // namespace

int make_plan(const ssm_dims_t* d, Plan* pl) {
  if (!d || !pl) return SSM_ERR_NULL_ARG;
  if (d->layout != SSM_LAYOUT_BDL && d->layout != SSM_LAYOUT_BLHP) return SSM_ERR_UNSUPPORTED;
  if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (d->discretization != SSM_DISC_DELTA_B && d->discretization != SSM_DISC_ZOH) return SSM_ERR_UNSUPPORTED;
  if (d->reserved != 0) return SSM_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->seqlen < 1 || d->dim < 1 || d->dstate < 1 || d->ngroups < 1) return SSM_ERR_BAD_DIMS;
  if (d->dstate > 256) return SSM_ERR_UNSUPPORTED;
  if (d->batch > 65535 || d->dim > (int64_t)1 << 30 || d->seqlen > ((int64_t)1 << 40)) return SSM_ERR_BAD_DIMS;
  int64_t rows_per_group, groups_or_heads;
  if (d->layout == SSM_LAYOUT_BDL) {
    if (d->dim % d->ngroups) return SSM_ERR_BAD_DIMS;
    rows_per_group = d->dim / d->ngroups;
    groups_or_heads = d->ngroups;
  } else {
    if (d->nheads < 1 || d->headdim < 1 || d->nheads > d->dim || d->headdim > d->dim) return SSM_ERR_BAD_DIMS;
    if (d->nheads * d->headdim != d->dim) return SSM_ERR_BAD_DIMS;   // no overflow: both <= dim <= 2^30
    if (d->nheads % d->ngroups) return SSM_ERR_BAD_DIMS;
    rows_per_group = d->headdim;
    groups_or_heads = d->nheads;
  }
  Plan p;
  p.disc = d->discretization;
  p.layout = d->layout;
  p.io = d->io_dtype;
  const int64_t N = d->dstate;
  p.Npad = N <= 16 ? 16 : N <= 32 ? 32 : N <= 64 ? 64 : N <= 128 ? 128 : 256;
  switch (p.Npad) {
    case 16: p.NS = 2; p.NW = 8; break;
    case 32: p.NS = 4; p.NW = 8; break;
    case 64: p.NS = 8; p.NW = 8; break;
    case 128: p.NS = 16; p.NW = 8; break;
    default: p.NS = 16; p.NW = 16; break;
  }
  // Per-channel layout with up to 32 states: one wave per 8 channels, no barriers.
  // (Its lane offsets along time are 32-bit: sequences up to 2^26 steps.)
  p.kernel = (d->layout == SSM_LAYOUT_BDL && p.Npad <= 32 && d->seqlen <= ((int64_t)1 << 26)) ? 1 : 0;
  int64_t units, target;
  if (p.kernel == 1) {
    p.NS = p.Npad / 8;
    p.NW = 1;
    p.TB = 32;
    p.blocks_per_group = (int)((rows_per_group + 7) / 8);
    const int64_t row_blocks = groups_or_heads * p.blocks_per_group;
    p.grid_rows = (int)((row_blocks + 3) / 4);
    units = row_blocks * d->batch;            // waves
    target = 4 * kCUs * 2;                    // two waves per SIMD
  } else {
    p.TB = 16;
    p.blocks_per_group = (int)((rows_per_group + 63) / 64);
    const int64_t grid_rows = groups_or_heads * p.blocks_per_group;
    if (grid_rows > 0x7fffffff) return SSM_ERR_BAD_DIMS;
    p.grid_rows = (int)grid_rows;
    units = grid_rows * d->batch;             // workgroups
    target = 2 * kCUs;
  }
  if ((int64_t)p.grid_rows > 0x7fffffff) return SSM_ERR_BAD_DIMS;
  // Multi-head layout in bfloat16 with 32/64/128 states: the chunked form on MFMA
  // (SSM_SCAN_SSD=0 keeps the scan kernel).
  const char* ssd_env = std::getenv("SSM_SCAN_SSD");
  const bool ssd_ok = !(ssd_env && *ssd_env == '0');
  if (ssd_ok && d->layout == SSM_LAYOUT_BLHP && d->io_dtype == SSM_BF16 && (N == 32 || N == 64 || N == 128) &&
      d->headdim % 16 == 0 && d->nheads <= 65535 &&
      64 * std::max<int64_t>(d->dim, d->ngroups * N) < ((int64_t)1 << 31)) {   // 32-bit offsets within a chunk
    p.kernel = 2;
    // positions per workgroup: 32 (two workgroups per CU), 16 when the head size needs it;
    // SSM_SSD_PS=16 forces 16 (tests, tuning)
    const char* ps_env = std::getenv("SSM_SSD_PS");
    p.ps = (d->headdim % 32 == 0 && !(ps_env && std::atoi(ps_env) == 16)) ? 32 : 16;
    p.NS = 0; p.NW = 4; p.TB = 64;
    p.grid_rows = (int)(d->headdim / p.ps);
    // time segments of whole 64-step chunks: an aggregate pass writes each segment's
    // zero-start end state and decay, the main pass folds them in.  About three workgroups
    // per CU (two are resident at a time): fewer leave CUs idle or half-loaded, more add
    // aggregate work (measured on 80 heads of 64 x 128 states, 8192 steps: 1, 2, 3, 4, 6
    // segments 0.56, 0.59, 0.49, 0.52, 0.52 ms for two sequences; one sequence 0.40 ->
    // 0.25 ms with 3).  Segments keep at least two chunks.  SSM_SCAN_SEGMENTS forces a count.
    p.nseg = 1;
    p.seg_len = d->seqlen;
    const int64_t ssd_wgs = (d->headdim / p.ps) * d->nheads * d->batch;
    int64_t ns = std::min<int64_t>((3 * kCUs + ssd_wgs - 1) / ssd_wgs, std::max<int64_t>(1, d->seqlen / 128));
    const char* seg_env = std::getenv("SSM_SCAN_SEGMENTS");
    if (seg_env && *seg_env) ns = std::atoi(seg_env);
    {
      ns = std::max<int64_t>(1, ns);
      int64_t len = round_up((d->seqlen + ns - 1) / ns, 64);
      ns = (d->seqlen + len - 1) / len;
      if (ns * d->batch <= 65535) {
        p.nseg = (int)ns;
        p.seg_len = len;
      }
    }
    p.vec_ok = true;
    p.bc_bytes = 0;
    // [seg][b][h] decays (padded to 256 bytes), then [seg][b][h][slice][tile][lane][4] states
    p.seg_bytes = p.nseg > 1 ? (size_t)round_up((int64_t)(p.nseg - 1) * d->batch * d->nheads * (int64_t)sizeof(float), 256) +
                                   (size_t)(p.nseg - 1) * (size_t)d->batch * (size_t)d->dim * (size_t)N * sizeof(float)
                             : 0;
    p.ws_bytes = p.seg_bytes;
    *pl = p;
    return SSM_OK;
  }
  p.nseg = choose_segments(d->seqlen, units, target, p.TB, &p.seg_len);
  p.vec_ok = (d->layout == SSM_LAYOUT_BDL) && (d->seqlen % 4 == 0);
  p.seg_bytes = p.nseg > 1 ? (size_t)2 * (size_t)(p.nseg - 1) * (size_t)d->batch * (size_t)p.Npad *
                                     (size_t)d->dim * sizeof(float)
                           : 0;
  if (p.kernel == 1) {
    p.nblk = (d->seqlen + p.TB - 1) / p.TB;
    if (p.nblk > 0x7fffffff) return SSM_ERR_BAD_DIMS;
    p.bc_bytes = (size_t)d->batch * (size_t)d->ngroups * (size_t)p.nblk * (size_t)p.TB * 2 * (size_t)p.Npad *
                 sizeof(float);
    p.bc_bytes = (p.bc_bytes + 255) & ~(size_t)255;
    // 16 states: a two-kind launch (one workgroup per CU per segment, the same channels on
    // every SIMD) when its busiest SIMD has less to do than the plain launch's, over the main
    // pass and (with time segments) the aggregate pass, which costs about 0.7 of a main pass
    // per step.  Two workgroup sizes: 80 channels (4 lanes x 4 states, and 16 lanes x 1
    // state; about 2.6 plain waves of work per SIMD) and 48 channels (8 lanes x 2 states,
    // and 16 x 1; about 1.9).  The 80-channel one picks its own segment count.  SSM_SCAN_MIXED=0 forces
    // the plain launch, 1 the 80-channel one, 48 the 48-channel one (tests, tuning).
    if (p.Npad == 16) {
      const char* seg_env = std::getenv("SSM_SCAN_SEGMENTS");
      const bool seg_forced = seg_env && *seg_env;
      const int64_t L = d->seqlen;
      auto pass_cost = [&](int64_t units, int64_t slots, int64_t nseg, double unit_cost) {
        const int64_t len = (int64_t)round_up((L + nseg - 1) / nseg, p.TB);
        const int64_t ns = (L + len - 1) / len;
        const double main = (double)((units * ns + slots - 1) / slots);
        const double agg = ns > 1 ? (double)((units * (ns - 1) + slots - 1) / slots) : 0.0;
        return unit_cost * (main + 0.7 * agg) * (double)len;
      };
      struct Cand {
        int64_t blocks, nseg;
        double cost;
      };
      auto candidate = [&](int64_t rows, double unit_cost, bool search) {
        Cand c;
        c.blocks = (rows_per_group + rows - 1) / rows;
        const int64_t wgs = c.blocks * groups_or_heads * d->batch;
        c.nseg = seg_forced ? p.nseg : 1;
        c.cost = pass_cost(wgs, kCUs, c.nseg, unit_cost);
        if (!seg_forced && search) {
          const int64_t max_seg = std::min<int64_t>(65535, (L + 255) / 256);
          for (int64_t ns = 2; ns <= std::min<int64_t>(max_seg, 64); ++ns) {
            const double cc = pass_cost(wgs, kCUs, ns, unit_cost);
            if (cc < c.cost) { c.cost = cc; c.nseg = ns; }
          }
        }
        return c;
      };
      const int64_t waves = (int64_t)p.blocks_per_group * groups_or_heads * d->batch;
      const double cost_plain = pass_cost(waves, 4 * kCUs, p.nseg, 1.0);
      // The 48-channel launch keeps one segment unless segments are forced: with its own
      // segment count it measured slower than either other launch on every shape tried.
      const Cand c80 = candidate(80, 2.6, true), c48 = candidate(48, 1.9, false);
      int rows = 0;   // 0: the plain launch
      if (c80.cost < cost_plain) rows = 80;
      if (c48.cost < std::min(cost_plain, c80.cost)) rows = 48;
      const char* env = std::getenv("SSM_SCAN_MIXED");
      if (env && *env) rows = *env == '0' ? 0 : std::atoi(env) == 48 ? 48 : 80;
      const Cand& c = rows == 48 ? c48 : c80;
      if (rows && groups_or_heads * c.blocks <= 0x7fffffff) {
        p.kernel = rows == 48 ? 6 : 5;
        if (p.kernel == 5) p.vec_ok = p.vec_ok && d->seqlen % 8 == 0;   // 8-step vectors
        p.blocks_per_group = (int)c.blocks;
        p.grid_rows = (int)(groups_or_heads * c.blocks);
        if (c.nseg != p.nseg) {   // the two-kind launch's own segment count
          int64_t len = round_up((L + c.nseg - 1) / c.nseg, p.TB);
          p.seg_len = len;
          p.nseg = (int)((L + len - 1) / len);
          p.seg_bytes = p.nseg > 1 ? (size_t)2 * (size_t)(p.nseg - 1) * (size_t)d->batch * (size_t)p.Npad *
                                         (size_t)d->dim * sizeof(float)
                                   : 0;
        }
      }
    }
  }
  p.ws_bytes = p.bc_bytes + p.seg_bytes;
  *pl = p;
  return SSM_OK;
}

int launch_plan(const Plan& plan, const KParams& kp, void* stream) {
  if (plan.kernel == 2) return launch_ssd(kp, plan.ps, plan.disc == SSM_DISC_ZOH, stream);
  return plan.disc == SSM_DISC_ZOH ? launch_plan_zoh(plan, kp, stream) : launch_plan_delta_b(plan, kp, stream);
}

}  // namespace ssm

extern "C" {

int ssm_scan_version(void) { return 100; }

const char* ssm_strerror(int code) {
  switch (code) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL_ARG: return "a required pointer (u, delta, A, B, C, y, dims) is NULL";
    case SSM_ERR_BAD_DIMS: return "invalid dimensions (size <= 0, nheads*headdim != dim, or groups do not divide)";
    case SSM_ERR_UNSUPPORTED: return "unsupported layout, io dtype, or dstate outside 1..256";
    case SSM_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SSM_ERR_ALIAS: return "an output overlaps an input or the other output";
    case SSM_ERR_WORKSPACE: return "workspace is smaller than ssm_scan_workspace_size()";
    case SSM_ERR_HIP: return ssm::g_hip_msg[0] ? ssm::g_hip_msg : "HIP runtime error";
    case SSM_ERR_SCRATCH:
      return "the launch needs more scratch than the static device scratch of ssm_scan_fwd_noalloc holds "
             "(ssm_scan_scratch_capacity() bytes)";
    default: return "unknown error code";
  }
}

size_t ssm_scan_workspace_size(const ssm_dims_t* dims) {
  ssm::Plan p;
  if (ssm::make_plan(dims, &p) != SSM_OK) return 0;
  return p.ws_bytes;
}

int ssm_scan_describe(const ssm_dims_t* dims, char* buf, size_t buf_len) {
  ssm::Plan p;
  const int rc = ssm::make_plan(dims, &p);
  if (rc != SSM_OK) return rc;
  if (buf && buf_len) {
    std::snprintf(buf, buf_len,
                  "kernel=%s layout=%s io=%s disc=%s NS=%d NW=%d TB=%d Npad=%d grid=(%d,%lld,%d) seg_len=%lld vec=%d "
                  "ws=%zu",
                  p.kernel == 6   ? "rowgroup_mixed48"
                  : p.kernel == 5 ? "rowgroup_mixed4"
                  : p.kernel == 2 ? "ssd"
                  : p.kernel == 1 ? "rowgroup"
                                  : "workgroup",
                  p.layout == SSM_LAYOUT_BDL ? "bdl" : "blhp",
                  p.io == SSM_BF16 ? "bf16" : "f32", p.disc == SSM_DISC_ZOH ? "zoh" : "delta_b", p.NS, p.NW, p.TB,
                  p.Npad, p.grid_rows, (long long)dims->batch, p.nseg, (long long)p.seg_len, (int)p.vec_ok,
                  p.ws_bytes);
  }
  return SSM_OK;
}

// use_scratch: the allocation-free variant (the library's static device scratch replaces the
// workspace; no allocation of any kind).
static int scan_entry(const void* u, const ssm_conv_t* conv, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias, int softplus_flag,
                      const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream,
                      bool use_scratch = false) {
  ssm::g_hip_msg[0] = 0;
  if (!u || !delta || !A || !B || !C || !y || !dims) return SSM_ERR_NULL_ARG;
  ssm::Plan pl;
  int rc = ssm::make_plan(dims, &pl);
  if (rc != SSM_OK) return rc;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, y, h_last};
  for (const void* q : ptrs)
    if (ssm::misaligned(q)) return SSM_ERR_ALIGN;
  if (conv) {
    if (!conv->weight) return SSM_ERR_NULL_ARG;
    if (conv->width < 1 || conv->width > 4 || conv->reserved != 0) return SSM_ERR_UNSUPPORTED;
    // the fused stage lives in the per-channel (row-group) kernels and the chunked multi-head kernel
    if (pl.kernel != 1 && pl.kernel != 5 && pl.kernel != 6 && pl.kernel != 2) return SSM_ERR_UNSUPPORTED;
    const void* cps[] = {conv->weight, conv->bias, conv->state_in, conv->state_out};
    for (const void* q : cps)
      if (ssm::misaligned(q)) return SSM_ERR_ALIGN;
  }

  // byte extents for the alias check
  const size_t esz = dims->io_dtype == SSM_BF16 ? 2 : 4;
  const size_t Bn = (size_t)dims->batch, L = (size_t)dims->seqlen, Dm = (size_t)dims->dim;
  const size_t N = (size_t)dims->dstate, G = (size_t)dims->ngroups;
  const bool bdl = dims->layout == SSM_LAYOUT_BDL;
  const size_t Hn = bdl ? Dm : (size_t)dims->nheads;
  const size_t n_x = Bn * Dm * L * esz;
  const size_t n_dt = (bdl ? Bn * Dm * L : Bn * L * Hn) * esz;
  const size_t n_bc = Bn * G * N * L * esz;
  const size_t n_A = (bdl ? Dm * N : Hn) * 4;
  const size_t n_bias = Hn * 4, n_D = Dm * 4, n_state = Bn * Dm * N * 4;
  struct Range { const void* p; size_t n; };
  const Range inputs[] = {{u, n_x}, {delta, n_dt}, {A, n_A}, {B, n_bc}, {C, n_bc},
                          {D, n_D}, {z, n_x}, {delta_bias, n_bias}, {h0, n_state}};
  for (const Range& r : inputs) {
    if (ssm::overlaps(y, n_x, r.p, r.n)) return SSM_ERR_ALIAS;
    if (ssm::overlaps(h_last, n_state, r.p, r.n)) return SSM_ERR_ALIAS;
  }
  if (ssm::overlaps(y, n_x, h_last, n_state)) return SSM_ERR_ALIAS;
  if (conv && conv->state_out) {
    const size_t K1 = (size_t)(conv->width - 1);
    const size_t n_cs = Bn * Dm * K1 * 4, n_w = Dm * (size_t)conv->width * 4;
    const Range more[] = {{conv->weight, n_w}, {conv->bias, Dm * 4}, {conv->state_in, n_cs}, {y, n_x},
                          {h_last, n_state}};
    for (const Range& r : inputs)
      if (ssm::overlaps(conv->state_out, n_cs, r.p, r.n)) return SSM_ERR_ALIAS;
    for (const Range& r : more)
      if (ssm::overlaps(conv->state_out, n_cs, r.p, r.n)) return SSM_ERR_ALIAS;
  }
  if (conv) {
    const Range cin[] = {{conv->weight, Dm * (size_t)conv->width * 4}, {conv->bias, Dm * 4},
                         {conv->state_in, Bn * Dm * (size_t)(conv->width - 1) * 4}};
    for (const Range& r : cin) {
      if (ssm::overlaps(y, n_x, r.p, r.n)) return SSM_ERR_ALIAS;
      if (ssm::overlaps(h_last, n_state, r.p, r.n)) return SSM_ERR_ALIAS;
    }
  }

  void* ws = use_scratch ? nullptr : dims->workspace;
  bool own_ws = false;
  if (use_scratch && pl.ws_bytes) {
    if (pl.ws_bytes > ssm::scratch_capacity()) return SSM_ERR_SCRATCH;
    const int rs = ssm::scratch_address(&ws, ssm::g_hip_msg, sizeof ssm::g_hip_msg);
    if (rs != SSM_OK) return rs;
  }
  if (pl.ws_bytes && !use_scratch) {
    if (ws) {
      if (dims->workspace_bytes < pl.ws_bytes) return SSM_ERR_WORKSPACE;
      if (ssm::misaligned(ws)) return SSM_ERR_ALIGN;
    }
  }
  if (pl.ws_bytes && !ws) {
    hipError_t e = hipMallocAsync(&ws, pl.ws_bytes, (hipStream_t)stream);
    if (e != hipSuccess) {
      std::snprintf(ssm::g_hip_msg, sizeof ssm::g_hip_msg, "hipMallocAsync(%zu): %s", pl.ws_bytes,
                    hipGetErrorString(e));
      return SSM_ERR_HIP;
    }
    own_ws = true;
  }

  ssm::KParams kp{};
  kp.u = u; kp.delta = delta; kp.A = A; kp.B = B; kp.C = C; kp.D = D; kp.z = z; kp.bias = delta_bias;
  kp.h0 = h0; kp.y = y; kp.h_last = h_last;
  const size_t half = pl.seg_bytes / 2 / sizeof(float);
  kp.bct = pl.bc_bytes ? (float*)ws : nullptr;
  kp.nblk = pl.nblk;
  kp.wsP = pl.seg_bytes ? (float*)((char*)ws + pl.bc_bytes) : nullptr;
  kp.wsH = pl.seg_bytes ? kp.wsP + half : nullptr;
  if (pl.kernel == 2 && pl.seg_bytes) {   // chunked multi-head kernel: decays, then states
    kp.wsP = (float*)ws;
    kp.wsH = (float*)((char*)ws + ssm::round_up((int64_t)(pl.nseg - 1) * dims->batch * (int64_t)Hn * (int64_t)sizeof(float), 256));
  }
  kp.L = dims->seqlen; kp.seg_len = pl.seg_len; kp.nseg = pl.nseg;
  kp.batch = (int)dims->batch; kp.dim = (int)dims->dim; kp.N = (int)dims->dstate; kp.Npad = pl.Npad;
  kp.H = (int)Hn; kp.P = bdl ? 1 : (int)dims->headdim; kp.G = (int)dims->ngroups;
  kp.rows_per_group = bdl ? (int)(Dm / G) : (int)dims->headdim;
  kp.blocks_per_group = pl.blocks_per_group;
  kp.heads_per_group = bdl ? 1 : (int)(Hn / G);
  kp.softplus = softplus_flag ? 1 : 0;
  kp.zsrc = z ? z : u;
  kp.has_z = z ? 1 : 0;
  kp.vec_ok = pl.vec_ok ? 1 : 0;
  if (conv) {
    kp.conv_w = conv->weight;
    kp.conv_b = conv->bias;
    kp.conv_sin = conv->state_in;
    kp.conv_sout = conv->state_out;
    kp.conv_k = conv->width;
  }

  const int he = ssm::launch_plan(pl, kp, stream);
  if (own_ws) {
    hipError_t e = hipFreeAsync(ws, (hipStream_t)stream);
    if (he == 0 && e != hipSuccess) {
      std::snprintf(ssm::g_hip_msg, sizeof ssm::g_hip_msg, "hipFreeAsync: %s", hipGetErrorString(e));
      return SSM_ERR_HIP;
    }
  }
  if (he != 0) {
    std::snprintf(ssm::g_hip_msg, sizeof ssm::g_hip_msg, "kernel launch: %s", hipGetErrorString((hipError_t)he));
    return SSM_ERR_HIP;
  }
  return SSM_OK;
}

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* delta_bias, int softplus_flag,
                 const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream) {
  return scan_entry(u, nullptr, delta, A, B, C, D, z, delta_bias, softplus_flag, h0, y, h_last, dims, stream);
}

int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int softplus_flag,
                         const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream) {
  return scan_entry(u, nullptr, delta, A, B, C, D, z, delta_bias, softplus_flag, h0, y, h_last, dims, stream, true);
}

size_t ssm_scan_scratch_capacity(void) { return ssm::scratch_capacity(); }

int ssm_conv_scan_fwd(const void* x, const ssm_conv_t* conv, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias, int softplus_flag,
                      const float* h0, void* y, float* h_last, const ssm_dims_t* dims, void* stream) {
  if (!conv) return SSM_ERR_NULL_ARG;
  return scan_entry(x, conv, delta, A, B, C, D, z, delta_bias, softplus_flag, h0, y, h_last, dims, stream);
}

int ssm_state_update(const void* x, const void* delta, const float* A, const void* B, const void* C,
                     const float* D, const void* z, const float* delta_bias, int softplus_flag,
                     const float* h_in, float* h_out, void* y, const ssm_dims_t* dims, void* stream) {
  ssm::g_hip_msg[0] = 0;
  if (!x || !delta || !A || !B || !C || !y || !dims) return SSM_ERR_NULL_ARG;
  ssm::Plan pl;
  int rc = ssm::make_plan(dims, &pl);
  if (rc != SSM_OK) return rc;
  if (dims->seqlen != 1) return SSM_ERR_BAD_DIMS;
  const void* ptrs[] = {x, delta, A, B, C, D, z, delta_bias, h_in, h_out, y};
  for (const void* q : ptrs)
    if (ssm::misaligned(q)) return SSM_ERR_ALIGN;

  const size_t esz = dims->io_dtype == SSM_BF16 ? 2 : 4;
  const size_t Bn = (size_t)dims->batch, Dm = (size_t)dims->dim, N = (size_t)dims->dstate;
  const size_t G = (size_t)dims->ngroups;
  const bool bdl = dims->layout == SSM_LAYOUT_BDL;
  const size_t Hn = bdl ? Dm : (size_t)dims->nheads;
  const size_t n_x = Bn * Dm * esz, n_dt = Bn * Hn * esz, n_bc = Bn * G * N * esz;
  const size_t n_A = (bdl ? Dm * N : Hn) * 4, n_bias = Hn * 4, n_D = Dm * 4, n_state = Bn * Dm * N * 4;
  struct Range { const void* p; size_t n; };
  const Range inputs[] = {{x, n_x}, {delta, n_dt}, {A, n_A}, {B, n_bc}, {C, n_bc},
                          {D, n_D}, {z, n_x}, {delta_bias, n_bias}, {h_in, n_state}};
  for (const Range& r : inputs) {
    if (ssm::overlaps(y, n_x, r.p, r.n)) return SSM_ERR_ALIAS;
    // the state may be updated in place (h_out == h_in exactly), never partially overlapped
    if (r.p == h_in && h_out == h_in) continue;
    if (ssm::overlaps(h_out, n_state, r.p, r.n)) return SSM_ERR_ALIAS;
  }
  if (ssm::overlaps(y, n_x, h_out, n_state)) return SSM_ERR_ALIAS;

  ssm::UParams up{};
  up.x = x; up.delta = delta; up.A = A; up.B = B; up.C = C; up.D = D; up.z = z; up.bias = delta_bias;
  up.h_in = h_in; up.h_out = h_out; up.y = y;
  up.rows = (int64_t)Bn * (int64_t)Dm;
  up.dim = (int)Dm; up.N = (int)N; up.H = (int)Hn; up.P = bdl ? 1 : (int)dims->headdim; up.G = (int)G;
  up.rows_per_group = bdl ? (int)(Dm / G) : (int)dims->headdim;
  up.heads_per_group = bdl ? 1 : (int)(Hn / G);
  up.softplus = softplus_flag ? 1 : 0;
  up.zoh = dims->discretization == SSM_DISC_ZOH ? 1 : 0;
  const int he = ssm::launch_update(up, dims->layout, dims->io_dtype, pl.Npad, stream);
  if (he != 0) {
    std::snprintf(ssm::g_hip_msg, sizeof ssm::g_hip_msg, "kernel launch: %s", hipGetErrorString((hipError_t)he));
    return SSM_ERR_HIP;
  }
  return SSM_OK;
}

}  // extern "C"
