// kernels.hpp -- argument blocks and launchers shared by the C-ABI layer
// (ssm_api.cpp) and the HIP kernel files.  Sizes here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Steps between two saved chunk-boundary states (the forward writes the state
// before every multiple of this step; the backward recomputes a chunk's
// states into registers, so a chunk must fit there).
constexpr int64_t kChunkLen = 32;

// Option bits (the flags argument of the *_ex entry points).
constexpr int kFlagZoh = 1;           // exact zero-order-hold input term
constexpr int kFlagReverse = 2;       // scan from the last step to the first
constexpr int kFlagDeltaPerToken = 4; // delta is (B, L), shared by all channels
constexpr int kFlagAccumulate = 8;    // forward only: y += result instead of y = result

// Widest causal convolution that can be fused in front of the scan.
constexpr int kMaxConv = 4;

struct FwdArgs {
  int64_t B, L, D, N;
  const void *u, *delta, *Bm, *Cm, *z;
  const float *A, *Dskip, *bias, *h0;
  int softplus;
  int flags;
  float *h_final;
  void *y;
  float *chunk_states;
  void *workspace;
  int64_t workspace_bytes;
  // sequence split (set by the launcher): segment length in steps (0 = one
  // segment; the first pass gets the length of its pieces), the local end
  // states and summed step sizes of the first pass's segments or pieces
  // ((B, rows, D, N) and (B, rows, D), rows = ceil(L / that length)), and the
  // true states entering each segment ((B, nseg, D, N)); fp32, in the workspace
  int64_t seg_len;
  float *seg_hloc, *seg_dsum, *seg_state;
  // causal depthwise convolution + SiLU producing u from x (conv_k = 0: u is given)
  const void *x;
  const float *conv_w, *conv_b;
  int conv_k;
};

struct BwdArgs {
  int64_t B, L, D, N;
  const void *u, *delta, *Bm, *Cm, *z, *dy;
  const float *A, *Dskip, *bias, *h0, *chunk_states, *dh_final;
  int softplus;
  int flags;
  void *du, *ddelta, *dB, *dC, *dz;
  float *dA, *dD, *dbias, *dh0;
  void *workspace;
  int64_t workspace_bytes;
  // convolution in front of the scan (conv_k = 0: none): u is recomputed from
  // x; the outputs are dx (in place of du), dconv_w and dconv_b
  const void *x;
  const float *conv_w, *conv_b;
  int conv_k;
  void *dx;
  float *dconv_w, *dconv_b;
};

struct DecodeArgs {
  int64_t B, D, N;
  float *state;
  const void *u, *delta, *Bm, *Cm, *z;
  const float *A, *Dskip, *bias;
  int softplus;
  int flags;
  void *y;
};

// Launch plan of a forward call (kernel kind, channels per workgroup,
// sequence split), as the launcher follows it on the current device.
constexpr int kPlanAllPurpose = 0;       // fwd_kernel: every phase on every wave
constexpr int kPlanWaveSpecialised = 1;  // fwd_ws_kernel: recurrence and service waves
struct FwdPlan {
  int kernel;
  int tile_channels;
  int64_t segments;     // 1 = no sequence split
  int64_t segment_len;  // steps per segment (0 = no split)
  int64_t first_pass_len;  // steps per piece of the split's first pass (0 = no split)
};
FwdPlan plan_fwd(const FwdArgs &a, int io_dtype);

// Bytes of the static scratch array the allocation-free forward uses in place
// of a workspace (the largest forward workspace it accepts).
constexpr int64_t kNoAllocScratchBytes = (int64_t)16 << 20;

// Device address of that array on the current device (looked up once per
// device; the array itself lives in scan_fwd.hip).
hipError_t noalloc_scratch(void **ptr);

// Scan of affine maps along rows: h[r, i] = a[r, i] h[r, i-1] + b[r, i] in scan
// order (from the last element to the first if reverse), from h0[r] (0 if
// null).  All (rows, len) fp32, row-major.
struct AffineScanArgs {
  int64_t rows, len;
  const float *a, *b, *h0;
  float *h;
  int reverse;
};
hipError_t launch_affine_scan(const AffineScanArgs &a, hipStream_t stream);

int64_t fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int io_dtype);
int64_t bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int io_dtype);
int64_t bwd_conv_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int io_dtype);

// Each launcher enqueues its kernels on `stream` and returns the first HIP
// error reported while enqueuing (hipSuccess otherwise).
hipError_t launch_fwd(const FwdArgs &a, int io_dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs &a, int io_dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int io_dtype, hipStream_t stream);

}  // namespace ssm
