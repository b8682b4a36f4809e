// ssm_api.cpp -- the extern "C" entry points declared in include/ssm_scan.h:
// argument validation (before anything is enqueued), size queries, error
// reporting, and dispatch to the HIP launchers.  No device code lives here.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/ssm_scan.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void *p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

bool valid_dstate(int64_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

// Largest element count any single tensor may have: offsets are 64-bit, and
// byte sizes must also fit.
constexpr int64_t kMaxElems = (int64_t)1 << 60;

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  if (a > 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return *out <= kMaxElems;
}

int check_sizes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype) {
  if (batch < 1 || seqlen < 1 || dim < 1 || dstate < 1)
    return fail(SSM_ERR_BAD_SHAPE, "sizes must be >= 1 (batch=%lld seqlen=%lld dim=%lld dstate=%lld)",
                (long long)batch, (long long)seqlen, (long long)dim, (long long)dstate);
  int64_t bl, bld, bln;
  if (!mul_ok(batch, seqlen, &bl) || !mul_ok(bl, dim, &bld) || !mul_ok(bl, dstate, &bln))
    return fail(SSM_ERR_BAD_SHAPE, "sizes overflow 64-bit element offsets");
  if (batch > 0x7fffffff)  // batch rows are a grid dimension of every launch
    return fail(SSM_ERR_UNSUPPORTED, "batch=%lld exceeds 2^31-1", (long long)batch);
  if (dim > ((int64_t)1 << 36))  // channel tiles (and the decode's lanes) of a row are a grid dimension
    return fail(SSM_ERR_UNSUPPORTED, "dim=%lld exceeds 2^36", (long long)dim);
  if (!valid_dstate(dstate))
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld not in {1,2,4,8,16}", (long long)dstate);
  if (dim % 8 != 0) return fail(SSM_ERR_UNSUPPORTED, "dim=%lld is not a multiple of 8", (long long)dim);
  if (io_dtype != SSM_F32 && io_dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "io_dtype=%d is neither SSM_F32 (0) nor SSM_BF16 (1)", io_dtype);
  return SSM_OK;
}

struct Ptr {
  const char *name;
  const void *p;
  bool required;
};

int check_ptrs(const Ptr *ps, int n) {
  for (int i = 0; i < n; ++i) {
    if (ps[i].required && ps[i].p == nullptr) return fail(SSM_ERR_NULL_ARG, "%s is NULL", ps[i].name);
    if (!aligned16(ps[i].p)) return fail(SSM_ERR_ALIGNMENT, "%s is not 16-byte aligned", ps[i].name);
  }
  return SSM_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return SSM_OK;
  return fail(SSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

const char *ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL_ARG: return "null argument";
    case SSM_ERR_BAD_SHAPE: return "bad shape";
    case SSM_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSM_ERR_ALIGNMENT: return "misaligned pointer";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *ssm_last_error(void) { return g_last_error; }

int64_t ssm_scan_chunk_len(void) { return ssm::kChunkLen; }

int64_t ssm_scan_chunk_states_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (check_sizes(batch, seqlen, dim, dstate, SSM_F32) != SSM_OK) return -1;
  const int64_t K = (seqlen + ssm::kChunkLen - 1) / ssm::kChunkLen;
  return batch * K * dim * dstate * 4;
}

int64_t ssm_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                     int io_dtype) {
  if (check_sizes(batch, seqlen, dim, dstate, io_dtype) != SSM_OK) return -1;
  return ssm::fwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
}

int64_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                     int io_dtype) {
  if (check_sizes(batch, seqlen, dim, dstate, io_dtype) != SSM_OK) return -1;
  return ssm::bwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
}

int ssm_scan_fwd_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                      int flags, int conv_width, ssm_fwd_plan *plan) {
  g_last_error[0] = 0;
  int st = check_sizes(batch, seqlen, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  if (plan == nullptr) return fail(SSM_ERR_NULL_ARG, "plan is NULL");
  if (flags & ~(SSM_FLAG_ZOH | SSM_FLAG_REVERSE | SSM_FLAG_DELTA_PER_TOKEN | SSM_FLAG_ACCUMULATE))
    return fail(SSM_ERR_UNSUPPORTED, "unknown flags 0x%x for the forward scan", flags);
  if (conv_width < 0 || conv_width > ssm::kMaxConv)
    return fail(SSM_ERR_UNSUPPORTED, "conv_width=%d not in 0..%d", conv_width, ssm::kMaxConv);
  if (conv_width && (flags & SSM_FLAG_REVERSE))
    return fail(SSM_ERR_UNSUPPORTED, "the fused convolution runs forward in time only");
  ssm::FwdArgs a{};
  a.B = batch, a.L = seqlen, a.D = dim, a.N = dstate, a.flags = flags, a.conv_k = conv_width;
  const ssm::FwdPlan p = ssm::plan_fwd(a, io_dtype);
  plan->kernel = p.kernel;
  plan->tile_channels = p.tile_channels;
  plan->segments = p.segments;
  plan->segment_len = p.segment_len;
  plan->first_pass_len = p.first_pass_len;
  return SSM_OK;
}

int ssm_affine_scan(int64_t rows, int64_t len, const float *a, const float *b, const float *h0,
                    float *h, int reverse, void *hip_stream) {
  g_last_error[0] = 0;
  if (rows < 1 || len < 1)
    return fail(SSM_ERR_BAD_SHAPE, "rows=%lld and len=%lld must be >= 1", (long long)rows, (long long)len);
  int64_t n;
  if (!mul_ok(rows, len, &n)) return fail(SSM_ERR_BAD_SHAPE, "rows * len overflows 64-bit offsets");
  if (rows > 4 * (int64_t)0x7fffffff)  // four rows per workgroup, workgroups are a grid dimension
    return fail(SSM_ERR_UNSUPPORTED, "rows=%lld exceeds 4 * (2^31 - 1)", (long long)rows);
  if (reverse != 0 && reverse != 1) return fail(SSM_ERR_UNSUPPORTED, "reverse=%d is neither 0 nor 1", reverse);
  const Ptr ps[] = {{"a", a, true}, {"b", b, true}, {"h", h, true}, {"h0", h0, false}};
  for (const Ptr &q : ps) {
    if (q.required && q.p == nullptr) return fail(SSM_ERR_NULL_ARG, "%s is NULL", q.name);
    if (((uintptr_t)q.p & 3u) != 0) return fail(SSM_ERR_ALIGNMENT, "%s is not 4-byte aligned", q.name);
  }
  ssm::AffineScanArgs args{rows, len, a, b, h0, h, reverse};
  return hip_status(ssm::launch_affine_scan(args, (hipStream_t)hip_stream), "ssm_affine_scan launch");
}

int ssm_scan_fwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                    const void *u, const void *delta, const float *A, const void *Bmat,
                    const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                    int delta_softplus, const float *h0, float *h_final, void *y,
                    float *chunk_states, void *workspace, int64_t workspace_bytes,
                    void *hip_stream, int flags) {
  g_last_error[0] = 0;
  int st = check_sizes(batch, seqlen, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  if (flags & ~(SSM_FLAG_ZOH | SSM_FLAG_REVERSE | SSM_FLAG_DELTA_PER_TOKEN | SSM_FLAG_ACCUMULATE))
    return fail(SSM_ERR_UNSUPPORTED, "unknown flags 0x%x for the forward scan", flags);
  const Ptr ps[] = {{"u", u, true},          {"delta", delta, true},   {"A", A, true},
                    {"Bmat", Bmat, true},    {"Cmat", Cmat, true},     {"y", y, true},
                    {"Dskip", Dskip, false}, {"z", z, false},          {"delta_bias", delta_bias, false},
                    {"h0", h0, false},       {"h_final", h_final, false},
                    {"chunk_states", chunk_states, false}, {"workspace", workspace, false}};
  st = check_ptrs(ps, (int)(sizeof(ps) / sizeof(ps[0])));
  if (st != SSM_OK) return st;
  const int64_t need = ssm::fwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SSM_ERR_WORKSPACE, "forward needs %lld workspace bytes, got %lld", (long long)need,
                (long long)(workspace ? workspace_bytes : 0));
  ssm::FwdArgs a{};
  a.B = batch, a.L = seqlen, a.D = dim, a.N = dstate;
  a.u = u, a.delta = delta, a.Bm = Bmat, a.Cm = Cmat, a.z = z;
  a.A = A, a.Dskip = Dskip, a.bias = delta_bias, a.h0 = h0;
  a.softplus = delta_softplus != 0, a.flags = flags;
  a.h_final = h_final, a.y = y, a.chunk_states = chunk_states;
  a.workspace = workspace, a.workspace_bytes = workspace_bytes;
  return hip_status(ssm::launch_fwd(a, io_dtype, (hipStream_t)hip_stream), "ssm_scan_fwd launch");
}

int ssm_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                         const void *u, const void *delta, const float *A, const void *Bmat,
                         const void *Cmat, const float *Dskip, const void *z,
                         const float *delta_bias, int delta_softplus, const float *h0,
                         float *h_final, void *y, float *chunk_states, void *hip_stream, int flags) {
  g_last_error[0] = 0;
  const int st = check_sizes(batch, seqlen, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  const int64_t need = ssm::fwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
  if (need > ssm::kNoAllocScratchBytes)
    return fail(SSM_ERR_WORKSPACE,
                "these sizes need %lld bytes of scratch; the allocation-free forward holds %lld "
                "(use ssm_scan_fwd_ex with a workspace)",
                (long long)need, (long long)ssm::kNoAllocScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    const int hs = hip_status(ssm::noalloc_scratch(&ws), "scratch address lookup");
    if (hs != SSM_OK) return hs;
  }
  return ssm_scan_fwd_ex(batch, seqlen, dim, dstate, io_dtype, u, delta, A, Bmat, Cmat, Dskip, z,
                         delta_bias, delta_softplus, h0, h_final, y, chunk_states, ws,
                         need > 0 ? ssm::kNoAllocScratchBytes : 0, hip_stream, flags);
}

int ssm_scan_fwd_conv(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                      const void *x, const float *conv_w, const float *conv_b, int conv_width,
                      const void *delta, const float *A, const void *Bmat, const void *Cmat,
                      const float *Dskip, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, float *h_final, void *y,
                      float *chunk_states, void *workspace, int64_t workspace_bytes,
                      void *hip_stream, int flags) {
  g_last_error[0] = 0;
  int st = check_sizes(batch, seqlen, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  if (flags & ~(SSM_FLAG_ZOH | SSM_FLAG_DELTA_PER_TOKEN | SSM_FLAG_ACCUMULATE))
    return fail(SSM_ERR_UNSUPPORTED, "flags 0x%x: the fused convolution runs forward in time only", flags);
  if (conv_width < 1 || conv_width > ssm::kMaxConv)
    return fail(SSM_ERR_UNSUPPORTED, "conv_width=%d not in 1..%d", conv_width, ssm::kMaxConv);
  const Ptr ps[] = {{"x", x, true},         {"conv_w", conv_w, true}, {"delta", delta, true},
                    {"A", A, true},         {"Bmat", Bmat, true},     {"Cmat", Cmat, true},
                    {"y", y, true},         {"conv_b", conv_b, false}, {"Dskip", Dskip, false},
                    {"z", z, false},        {"delta_bias", delta_bias, false}, {"h0", h0, false},
                    {"h_final", h_final, false}, {"chunk_states", chunk_states, false},
                    {"workspace", workspace, false}};
  st = check_ptrs(ps, (int)(sizeof(ps) / sizeof(ps[0])));
  if (st != SSM_OK) return st;
  const int64_t need = ssm::fwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SSM_ERR_WORKSPACE, "forward needs %lld workspace bytes, got %lld", (long long)need,
                (long long)(workspace ? workspace_bytes : 0));
  ssm::FwdArgs a{};
  a.B = batch, a.L = seqlen, a.D = dim, a.N = dstate;
  a.u = nullptr, a.delta = delta, a.Bm = Bmat, a.Cm = Cmat, a.z = z;
  a.A = A, a.Dskip = Dskip, a.bias = delta_bias, a.h0 = h0;
  a.softplus = delta_softplus != 0, a.flags = flags;
  a.h_final = h_final, a.y = y, a.chunk_states = chunk_states;
  a.workspace = workspace, a.workspace_bytes = workspace_bytes;
  a.x = x, a.conv_w = conv_w, a.conv_b = conv_b, a.conv_k = conv_width;
  return hip_status(ssm::launch_fwd(a, io_dtype, (hipStream_t)hip_stream), "ssm_scan_fwd_conv launch");
}

int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *Bmat,
                 const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                 int delta_softplus, const float *h0, float *h_final, void *y,
                 float *chunk_states, void *workspace, int64_t workspace_bytes,
                 void *hip_stream) {
  return ssm_scan_fwd_ex(batch, seqlen, dim, dstate, io_dtype, u, delta, A, Bmat, Cmat, Dskip, z,
                         delta_bias, delta_softplus, h0, h_final, y, chunk_states, workspace,
                         workspace_bytes, hip_stream, 0);
}

int ssm_scan_bwd_ex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                    const void *u, const void *delta, const float *A, const void *Bmat,
                    const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                    int delta_softplus, const float *h0, const float *chunk_states, const void *dy,
                    const float *dh_final, void *du, void *ddelta, float *dA, void *dB, void *dC,
                    float *dD, void *dz, float *ddelta_bias, float *dh0, void *workspace,
                    int64_t workspace_bytes, void *hip_stream, int flags) {
  g_last_error[0] = 0;
  int st = check_sizes(batch, seqlen, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  if (flags & ~(SSM_FLAG_ZOH | SSM_FLAG_REVERSE | SSM_FLAG_DELTA_PER_TOKEN))
    return fail(SSM_ERR_UNSUPPORTED, "unknown or forward-only flags 0x%x for the backward scan", flags);
  const Ptr ps[] = {{"u", u, true},
                    {"delta", delta, true},
                    {"A", A, true},
                    {"Bmat", Bmat, true},
                    {"Cmat", Cmat, true},
                    {"chunk_states", chunk_states, true},
                    {"dy", dy, true},
                    {"du", du, true},
                    {"ddelta", ddelta, true},
                    {"dA", dA, true},
                    {"dB", dB, true},
                    {"dC", dC, true},
                    {"workspace", workspace, true},
                    {"Dskip", Dskip, false},
                    {"z", z, false},
                    {"delta_bias", delta_bias, false},
                    {"h0", h0, false},
                    {"dh_final", dh_final, false},
                    {"dD", dD, false},
                    {"dz", dz, false},
                    {"ddelta_bias", ddelta_bias, false},
                    {"dh0", dh0, false}};
  st = check_ptrs(ps, (int)(sizeof(ps) / sizeof(ps[0])));
  if (st != SSM_OK) return st;
  if ((Dskip == nullptr) != (dD == nullptr))
    return fail(SSM_ERR_NULL_ARG, "dD must be given if and only if Dskip is");
  if ((z == nullptr) != (dz == nullptr))
    return fail(SSM_ERR_NULL_ARG, "dz must be given if and only if z is");
  const int64_t need = ssm::bwd_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
  if (workspace_bytes < need)
    return fail(SSM_ERR_WORKSPACE, "backward needs %lld workspace bytes, got %lld", (long long)need,
                (long long)workspace_bytes);
  ssm::BwdArgs a{};
  a.B = batch, a.L = seqlen, a.D = dim, a.N = dstate;
  a.u = u, a.delta = delta, a.Bm = Bmat, a.Cm = Cmat, a.z = z, a.dy = dy;
  a.A = A, a.Dskip = Dskip, a.bias = delta_bias, a.h0 = h0, a.chunk_states = chunk_states;
  a.dh_final = dh_final, a.softplus = delta_softplus != 0, a.flags = flags;
  a.du = du, a.ddelta = ddelta, a.dB = dB, a.dC = dC, a.dz = dz;
  a.dA = dA, a.dD = dD, a.dbias = ddelta_bias, a.dh0 = dh0;
  a.workspace = workspace, a.workspace_bytes = workspace_bytes;
  return hip_status(ssm::launch_bwd(a, io_dtype, (hipStream_t)hip_stream), "ssm_scan_bwd launch");
}

int64_t ssm_scan_bwd_conv_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                          int io_dtype) {
  if (check_sizes(batch, seqlen, dim, dstate, io_dtype) != SSM_OK) return -1;
  return ssm::bwd_conv_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
}

int ssm_scan_bwd_conv(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                      const void *x, const float *conv_w, const float *conv_b, int conv_width,
                      const void *delta, const float *A, const void *Bmat, const void *Cmat,
                      const float *Dskip, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, const float *chunk_states,
                      const void *dy, const float *dh_final, void *dx, float *dconv_w,
                      float *dconv_b, void *ddelta, float *dA, void *dB, void *dC, float *dD,
                      void *dz, float *ddelta_bias, float *dh0, void *workspace,
                      int64_t workspace_bytes, void *hip_stream, int flags) {
  g_last_error[0] = 0;
  int st = check_sizes(batch, seqlen, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  if (flags & ~(SSM_FLAG_ZOH | SSM_FLAG_DELTA_PER_TOKEN))
    return fail(SSM_ERR_UNSUPPORTED, "flags 0x%x not supported with the fused convolution backward", flags);
  if (conv_width < 1 || conv_width > ssm::kMaxConv)
    return fail(SSM_ERR_UNSUPPORTED, "conv_width=%d not in 1..%d", conv_width, ssm::kMaxConv);
  const Ptr ps[] = {{"x", x, true},           {"conv_w", conv_w, true},    {"delta", delta, true},
                    {"A", A, true},           {"Bmat", Bmat, true},        {"Cmat", Cmat, true},
                    {"chunk_states", chunk_states, true}, {"dy", dy, true}, {"dx", dx, true},
                    {"dconv_w", dconv_w, true}, {"ddelta", ddelta, true},  {"dA", dA, true},
                    {"dB", dB, true},         {"dC", dC, true},            {"workspace", workspace, true},
                    {"conv_b", conv_b, false}, {"dconv_b", dconv_b, false}, {"Dskip", Dskip, false},
                    {"z", z, false},          {"delta_bias", delta_bias, false}, {"h0", h0, false},
                    {"dh_final", dh_final, false}, {"dD", dD, false},      {"dz", dz, false},
                    {"ddelta_bias", ddelta_bias, false}, {"dh0", dh0, false}};
  st = check_ptrs(ps, (int)(sizeof(ps) / sizeof(ps[0])));
  if (st != SSM_OK) return st;
  if ((conv_b == nullptr) != (dconv_b == nullptr))
    return fail(SSM_ERR_NULL_ARG, "dconv_b must be given if and only if conv_b is");
  if ((Dskip == nullptr) != (dD == nullptr))
    return fail(SSM_ERR_NULL_ARG, "dD must be given if and only if Dskip is");
  if ((z == nullptr) != (dz == nullptr))
    return fail(SSM_ERR_NULL_ARG, "dz must be given if and only if z is");
  const int64_t need = ssm::bwd_conv_workspace_bytes(batch, seqlen, dim, dstate, io_dtype);
  if (workspace_bytes < need)
    return fail(SSM_ERR_WORKSPACE, "backward with convolution needs %lld workspace bytes, got %lld",
                (long long)need, (long long)workspace_bytes);
  ssm::BwdArgs a{};
  a.B = batch, a.L = seqlen, a.D = dim, a.N = dstate;
  a.u = nullptr, a.delta = delta, a.Bm = Bmat, a.Cm = Cmat, a.z = z, a.dy = dy;
  a.A = A, a.Dskip = Dskip, a.bias = delta_bias, a.h0 = h0, a.chunk_states = chunk_states;
  a.dh_final = dh_final, a.softplus = delta_softplus != 0, a.flags = flags;
  a.du = nullptr, a.ddelta = ddelta, a.dB = dB, a.dC = dC, a.dz = dz;
  a.dA = dA, a.dD = dD, a.dbias = ddelta_bias, a.dh0 = dh0;
  a.workspace = workspace, a.workspace_bytes = workspace_bytes;
  a.x = x, a.conv_w = conv_w, a.conv_b = conv_b, a.conv_k = conv_width;
  a.dx = dx, a.dconv_w = dconv_w, a.dconv_b = dconv_b;
  return hip_status(ssm::launch_bwd(a, io_dtype, (hipStream_t)hip_stream), "ssm_scan_bwd_conv launch");
}

int ssm_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *Bmat,
                 const void *Cmat, const float *Dskip, const void *z, const float *delta_bias,
                 int delta_softplus, const float *h0, const float *chunk_states, const void *dy,
                 const float *dh_final, void *du, void *ddelta, float *dA, void *dB, void *dC,
                 float *dD, void *dz, float *ddelta_bias, float *dh0, void *workspace,
                 int64_t workspace_bytes, void *hip_stream) {
  return ssm_scan_bwd_ex(batch, seqlen, dim, dstate, io_dtype, u, delta, A, Bmat, Cmat, Dskip, z,
                         delta_bias, delta_softplus, h0, chunk_states, dy, dh_final, du, ddelta, dA,
                         dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes, hip_stream, 0);
}

int ssm_state_update_ex(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float *state,
                        const void *u, const void *delta, const float *A, const void *Bmat,
                        const void *Cmat, const float *Dskip, const void *z,
                        const float *delta_bias, int delta_softplus, void *y, void *hip_stream,
                        int flags) {
  g_last_error[0] = 0;
  int st = check_sizes(batch, 1, dim, dstate, io_dtype);
  if (st != SSM_OK) return st;
  if (flags & ~SSM_FLAG_ZOH)
    return fail(SSM_ERR_UNSUPPORTED, "only SSM_FLAG_ZOH applies to a single-token update (got 0x%x)", flags);
  // state and A are accessed 16 bytes at a time; the per-token tensors only
  // need the natural alignment of their element type.
  const Ptr ps[] = {{"state", state, true}, {"A", A, true}};
  st = check_ptrs(ps, 2);
  if (st != SSM_OK) return st;
  const size_t es = io_dtype == SSM_F32 ? 4 : 2;
  const Ptr tok[] = {{"u", u, true},       {"delta", delta, true},  {"Bmat", Bmat, true},
                     {"Cmat", Cmat, true}, {"y", y, true},          {"z", z, false},
                     {"Dskip", Dskip, false}, {"delta_bias", delta_bias, false}};
  for (const Ptr &q : tok) {
    if (q.required && q.p == nullptr) return fail(SSM_ERR_NULL_ARG, "%s is NULL", q.name);
    const size_t need = (q.p == Dskip || q.p == delta_bias) ? 4 : es;
    if (((uintptr_t)q.p % need) != 0)
      return fail(SSM_ERR_ALIGNMENT, "%s is not aligned to its element size", q.name);
  }
  ssm::DecodeArgs a{};
  a.B = batch, a.D = dim, a.N = dstate, a.state = state;
  a.u = u, a.delta = delta, a.Bm = Bmat, a.Cm = Cmat, a.z = z;
  a.A = A, a.Dskip = Dskip, a.bias = delta_bias, a.softplus = delta_softplus != 0, a.flags = flags;
  a.y = y;
  return hip_status(ssm::launch_decode(a, io_dtype, (hipStream_t)hip_stream), "ssm_state_update launch");
}

int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float *state,
                     const void *u, const void *delta, const float *A, const void *Bmat,
                     const void *Cmat, const float *Dskip, const void *z,
                     const float *delta_bias, int delta_softplus, void *y, void *hip_stream) {
  return ssm_state_update_ex(batch, dim, dstate, io_dtype, state, u, delta, A, Bmat, Cmat, Dskip, z,
                             delta_bias, delta_softplus, y, hip_stream, 0);
}

}  // extern "C"
