// state_update.hip -- one decode step of the selective SSM (reading guide of
// arXiv 2312.00752, "Sorular", question on KV caches: a fixed D x N state per
// layer advanced one token at a time).  The (B,D,N) fp32 state is streamed
// once in and once out with 16-byte accesses; everything else is small.
//
// Mapping: each lane owns SPL = min(N, 8) consecutive states of one channel,
// LPC = N / SPL lanes share a channel (adjacent lanes), so a wave reads and
// writes one contiguous 2 KiB span of the state.  The per-channel prologue is
// recomputed by the LPC lanes of the channel (cheaper than sharing it), the
// partial sum_n C h is reduced across them with cross-lane adds, and the first
// lane of the group stores y.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {

// States per lane.  Measured on MI355X for a (256, 5120, 16) fp32 state: 4
// per lane streams at 3.96 TB/s, 8 per lane (two 16-byte pieces in flight per
// lane) at 4.67 TB/s, 16 per lane at 3.66 TB/s; non-temporal accesses helped
// only the 4-per-lane layout.
constexpr int kDecodeSPL = 8;

// ZOH: exact zero-order-hold input term expm1(dt A)/A * B * u (reading
// guide, "Yöntem", discretisation of B) instead of dt * B * u.
template <typename IO, int N, bool ZOH>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
  constexpr int SPL = N < kDecodeSPL ? N : kDecodeSPL;  // states per lane
  constexpr int LPC = N / SPL;                          // lanes per channel
  constexpr int NV = SPL >= 4 ? SPL / 4 : 0;            // 16-byte pieces per lane
  // grid: x covers the channels of one batch row (LPC lanes each), y the rows
  // 64-bit: dim * LPC may exceed 2^31 lanes per batch row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t dd = gid / LPC;  // LPC is a power of two: shifts, not divisions
  const int g = (int)(gid % LPC);
  const bool valid = dd < a.D;
  const int64_t d = valid ? dd : 0;
  const int64_t chc = b * a.D + d;  // b * D + d
  const IO *u = (const IO *)a.u, *dl = (const IO *)a.delta, *zz = (const IO *)a.z;
  const IO *Bm = (const IO *)a.Bm, *Cm = (const IO *)a.Cm;

  float st[SPL], Av[SPL];
  float *sp = a.state + chc * N + g * SPL;
  if constexpr (NV > 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float4 q = ((const float4 *)sp)[v];
      st[4 * v] = q.x, st[4 * v + 1] = q.y, st[4 * v + 2] = q.z, st[4 * v + 3] = q.w;
      const float4 r = *((const float4 *)(a.A + d * N + g * SPL) + v);
      Av[4 * v] = r.x, Av[4 * v + 1] = r.y, Av[4 * v + 2] = r.z, Av[4 * v + 3] = r.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < SPL; ++k) st[k] = sp[k], Av[k] = a.A[d * N + g * SPL + k];
  }
  const float x = load_io(u, chc);
  const float dt = step_size(load_io(dl, chc), a.bias ? a.bias[d] : 0.0f, a.softplus != 0);
  const float dtu = dt * x;
  float ys = 0.0f;
#pragma unroll
  for (int k = 0; k < SPL; ++k) {
    const int64_t bn = b * N + g * SPL + k;
    const float da = fast_exp2(dt * Av[k] * kLog2e);
    if (ZOH) {
      const float cf = zoh_coef(dt, dt * Av[k], da, 1.0f / Av[k]);
      st[k] = fmaf(da, st[k], cf * x * load_io(Bm, bn));
    } else {
      st[k] = fmaf(da, st[k], dtu * load_io(Bm, bn));
    }
    ys = fmaf(load_io(Cm, bn), st[k], ys);
  }
#pragma unroll
  for (int off = 1; off < LPC; off <<= 1) ys += __shfl_xor(ys, off, 64);
  if (!valid) return;
  if constexpr (NV > 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      ((float4 *)sp)[v] = make_float4(st[4 * v], st[4 * v + 1], st[4 * v + 2], st[4 * v + 3]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < SPL; ++k) sp[k] = st[k];
  }
  if (g == 0) {
    float out = fmaf(a.Dskip ? a.Dskip[d] : 0.0f, x, ys);
    if (a.z) out *= silu_f(load_io(zz, chc));
    store_io((IO *)a.y, chc, out);
  }
}

template <typename IO, int N>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
  constexpr int LPC = N < kDecodeSPL ? 1 : N / kDecodeSPL;
  const int64_t threads = a.D * LPC;  // per batch row
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)a.B);
  if (a.flags & kFlagZoh)
    hipLaunchKernelGGL((decode_kernel<IO, N, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<IO, N, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_decode_io(const DecodeArgs &a, hipStream_t s) {
  switch (a.N) {
    case 1: return launch_decode_t<IO, 1>(a, s);
    case 2: return launch_decode_t<IO, 2>(a, s);
    case 4: return launch_decode_t<IO, 4>(a, s);
    case 8: return launch_decode_t<IO, 8>(a, s);
    case 16: return launch_decode_t<IO, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == 0 ? launch_decode_io<float>(a, s) : launch_decode_io<bf16>(a, s);
}

}  // namespace ssm
