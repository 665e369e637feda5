// scan_plan.h -- launch plan shared by the host API and the kernel launchers.
//
// A workgroup owns 64 "rows" (channels of one batch item: one channel group in the
// (B,D,L) layout, 64 positions of one head in the (B,L,H,P) layout) and all of their
// states.  The state index is split over NW waves with NS states per lane
// (NS*NW = Npad >= dstate; padded states carry A = B = C = 0 and stay zero).
// Time is walked in blocks of TB steps; a sequence may be cut into nseg time
// segments, in which case an aggregate pass computes each segment's decay product
// and zero-start end state, and the main pass folds them into its initial state.
#pragma once
#include <cstddef>
#include <cstdint>

#include "ssm_scan.h"

namespace ssm {

struct Plan {
  int kernel = 0;            // 0: workgroup kernel (64 rows, states over waves); 1: row-group kernel;
                             // 2: chunked multi-head kernel on MFMA (ssd_kernels.hip);
                             // 5 / 6: row-group kernel, two-kind launch (16 states, 80 / 48 channels
                             // per workgroup)
  int ps = 0;                // kernel 2: positions per workgroup
  int disc = 0;              // SSM_DISC_DELTA_B or SSM_DISC_ZOH
  int layout = 0, io = 0;
  int NS = 0, NW = 0, TB = 0, Npad = 0;
  int nseg = 1;
  int64_t seg_len = 0;
  int blocks_per_group = 0;  // row blocks per channel group (BDL) or per head (BLHP)
  int grid_rows = 0;         // workgroups per batch item and segment
  bool vec_ok = false;       // 4-step vector loads allowed along time (BDL)
  int64_t nblk = 0;          // row-group kernel: 32-step time blocks per sequence
  size_t bc_bytes = 0;       // row-group kernel: fp32 B/C tiles (start of the workspace)
  size_t seg_bytes = 0;      // segment aggregates (after the tiles)
  size_t ws_bytes = 0;       // total workspace
};

struct KParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const void* zsrc;     // z, or u when there is no gate (prefetched unconditionally, unused then)
  const float* bias;
  const float* h0;
  void* y;
  float* h_last;
  float* wsP;   // [seg][b][n][d] decay product of each aggregated segment ([seg][b][h] in the
                //   chunked multi-head kernel)
  float* wsH;   // [seg][b][n][d] zero-start end state of each aggregated segment ([seg][b][h]
                //   [slice][state tile][lane][4] in the chunked multi-head kernel)
  float* bct;   // row-group kernel: [b][g][block] B/C tiles in LDS order (bc_tile_kernel)
  const float* conv_w;     // optional input stage (row-group kernels): (dim, conv_k) filters
  const float* conv_b;     // (dim) or NULL
  const float* conv_sin;   // (batch, dim, conv_k-1) raw inputs before t = 0, or NULL (zeros)
  float* conv_sout;        // (batch, dim, conv_k-1) last raw inputs, or NULL
  int conv_k;              // 0: no input stage; 1..4: filter width
  int64_t nblk; // row-group kernel: time blocks per sequence
  int64_t L, seg_len;
  int batch, dim, N, Npad, H, P, G;
  int rows_per_group;    // BDL: dim / G;  BLHP: P
  int blocks_per_group;  // row blocks per group / head (64 rows; 8 for the row-group kernel; 80 or 48 for
                         // the two-kind launches)
  int heads_per_group;   // BLHP: H / G
  int softplus;
  int has_z;
  int vec_ok;
  int nseg;
};

// Arguments of the single-token state update (seqlen = 1).
struct UParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const float* h_in;
  float* h_out;
  void* y;
  int64_t rows;          // batch * dim
  int dim, N, H, P, G;
  int rows_per_group;    // BDL: dim / G
  int heads_per_group;   // BLHP: H / G
  int softplus;
  int zoh;               // exact zero-order hold for B̄
};

// Validates dims (no HIP call) and fills the plan; returns SSM_OK or an error code.
int make_plan(const ssm_dims_t* d, Plan* plan);

// Enqueue the kernels of a validated plan.  Returns a hipError_t value (0 = success).
// scan_kernels.hip is compiled once per discretization; launch_plan picks the build.
int launch_plan(const Plan& plan, const KParams& kp, void* stream);
int launch_plan_delta_b(const Plan& plan, const KParams& kp, void* stream);
int launch_plan_zoh(const Plan& plan, const KParams& kp, void* stream);

// Enqueue the chunked multi-head kernel (bf16 storage, N in {32,64,128}, ps in {32,64} dividing P).
int launch_ssd(const KParams& kp, int ps, int zoh, void* stream);

// Enqueue the state-update kernel.  Returns a hipError_t value (0 = success).
int launch_update(const UParams& p, int layout, int io, int Npad, void* stream);

// The static device scratch of the allocation-free entry point (scratch.hip): its size in
// bytes, and its device address on the current device (looked up once per device).
// scratch_address returns SSM_OK or SSM_ERR_HIP (with a message in msg).
size_t scratch_capacity();
int scratch_address(void** out, char* msg, size_t msg_len);

}  // namespace ssm
