// scan_fwd.hip -- forward selective scan for gfx950.
//
// Computes, per (b, d, n), the recurrence of the Mamba selective SSM
// (reading guide of arXiv 2312.00752, "Yöntem" and "Seçim Mekanizması (S6)"):
//   dt = softplus(delta + bias), h = exp(dt*A) h + dt*B*u,
//   y = (sum_n C h + D u) * silu(z)
// with the state held in registers and only y (B,L,D) written back (the
// "Donanım Duyarlı Durum Genişletme" section: the expanded state is never
// materialised in device memory).
//
// Mapping (one workgroup = 64 consecutive channels of one batch row):
//   - lanes <-> channels d, so every (B,L,D) access of a wave is 64
//     consecutive elements (coalesced);
//   - the N states of a channel are split over NW = N/NPL waves, NPL states
//     per lane, so that the 16-state problems put 2 waves on every SIMD;
//   - time is processed in chunks of T steps.  For each chunk, every thread
//     computes the per-(t,d) prologue (dt, dt*u) for T/NW of the steps once
//     and shares it through LDS; each wave then runs the recurrence for its
//     states over the T steps, reading B and C as wave-uniform scalar loads,
//     and leaves its partial sum_n C h in LDS; finally every thread reduces
//     the partials over waves for its steps, adds D*u, applies the gate and
//     stores y.  Global loads of the next chunk are issued before the
//     recurrence of the current one so they are in flight while it runs.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(4))) const float cfloat4_t;
typedef __attribute__((address_space(4))) const f32x2_t cfloat2_4_t;
typedef __attribute__((address_space(4))) const uint32_t cuint4_t;

// Wave-uniform loads of NPL consecutive values (B or C for a wave's states)
// through the scalar unit.  `i` is a multiple of NPL.
template <int NPL>
__device__ __forceinline__ void uniform_load(const float *p, int64_t i, float *out) {
  if constexpr (NPL == 2) {
    const f32x2_t v = ((cfloat2_4_t *)(p + i))[0];
    out[0] = v.x;
    out[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < NPL; ++k) out[k] = ((cfloat4_t *)p)[i + k];
  }
}
// bf16: for NPL = 2 the pair is one aligned dword (p + i is 4-byte aligned
// because N is even); a single bf16 value is read with an ordinary load.
template <int NPL>
__device__ __forceinline__ void uniform_load(const bf16 *p, int64_t i, float *out) {
  if constexpr (NPL == 2) {
    const uint32_t bits = ((cuint4_t *)(p + i))[0];
    out[0] = __uint_as_float(bits << 16);
    out[1] = __uint_as_float(bits & 0xffff0000u);
  } else {
#pragma unroll
    for (int k = 0; k < NPL; ++k) out[k] = load_io(p, i + k);
  }
}

template <typename IO, int N, int NPL, int T>
__global__ void __launch_bounds__(64 * (N / NPL)) fwd_chunked_kernel(FwdArgs a) {
  constexpr int NW = N / NPL;
  constexpr int TPW = T / NW;  // prologue/epilogue steps per thread per chunk
  static_assert(T % NW == 0, "chunk must split evenly over waves");
  const IO *__restrict__ u = (const IO *)a.u;
  const IO *__restrict__ dl = (const IO *)a.delta;
  const IO *__restrict__ zz = (const IO *)a.z;
  const IO *Bm = (const IO *)a.Bm;
  const IO *Cm = (const IO *)a.Cm;
  IO *__restrict__ y = (IO *)a.y;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t L = a.L, D = a.D;
  const int64_t b = blockIdx.y;
  const int64_t d = (int64_t)blockIdx.x * 64 + lane;
  const bool dv = d < D;
  const int64_t dc = dv ? d : D - 1;  // clamped channel for loads
  const bool has_z = a.z != nullptr;
  const bool sp = a.softplus != 0;

  __shared__ float2 P[T][64];        // (dt, dt*u) per step and channel
  __shared__ float Y[T][NW][64];     // per-wave partial sum_n C h

  float Ap[NPL], h[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int n = w * NPL + k;
    Ap[k] = a.A[dc * N + n] * kLog2e;
    h[k] = a.h0 ? a.h0[(b * D + dc) * N + n] : 0.0f;
  }
  const float bias = a.bias ? a.bias[dc] : 0.0f;
  const float Dv = a.Dskip ? a.Dskip[dc] : 0.0f;

  float r_raw[TPW], r_u[TPW], r_z[TPW];   // loads in flight for the next chunk
  float keep_u[TPW], keep_g[TPW];         // kept for the epilogue
  const int64_t row0 = b * L;
  const int64_t nck = (L + T - 1) / T;
  const int64_t K = (L + kChunkLen - 1) / kChunkLen;

  auto load_chunk = [&](int64_t k) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int64_t t = k * T + w * TPW + j;
      const int64_t idx = (row0 + (t < L ? t : L - 1)) * D + dc;
      r_raw[j] = load_io(dl, idx);
      r_u[j] = load_io(u, idx);
      r_z[j] = has_z ? load_io(zz, idx) : 0.0f;
    }
  };
  auto prologue = [&](int64_t k) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tl = w * TPW + j;
      const int64_t t = k * T + tl;
      float dt = 0.0f, dtu = 0.0f;  // steps past the end leave the state unchanged
      if (t < L) {
        dt = step_size(r_raw[j], bias, sp);
        dtu = dt * r_u[j];
      }
      P[tl][lane] = make_float2(dt, dtu);
      keep_u[j] = r_u[j];
      keep_g[j] = has_z ? silu_f(r_z[j]) : 1.0f;
    }
  };

  load_chunk(0);
  prologue(0);
  __syncthreads();
  for (int64_t k = 0; k < nck; ++k) {
    const int64_t t0 = k * T;
    if (a.chunk_states && (t0 % kChunkLen) == 0 && dv) {
      float *cs = a.chunk_states + ((b * K + t0 / kChunkLen) * D + d) * N + w * NPL;
#pragma unroll
      for (int kk = 0; kk < NPL; ++kk) cs[kk] = h[kk];
    }
    if (k + 1 < nck) load_chunk(k + 1);
    // B and C rows of this chunk for this wave's states; in a full chunk the
    // per-step offsets are constants, in the ragged last chunk they are
    // clamped to the last row (those steps have dt = 0 and change nothing).
    const IO *Bp = Bm + (row0 + t0) * N + w * NPL;
    const IO *Cp = Cm + (row0 + t0) * N + w * NPL;
    auto scan_steps = [&](auto full) {
#pragma unroll
      for (int tl = 0; tl < T; ++tl) {
        int64_t off = (int64_t)tl * N;
        if constexpr (!decltype(full)::value) {
          if (t0 + tl >= L) off = (L - 1 - t0) * N;
        }
        const float2 p = P[tl][lane];
        float Bv[NPL], Cv[NPL];
        uniform_load<NPL>(Bp, off, Bv);
        uniform_load<NPL>(Cp, off, Cv);
        float ys = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NPL; ++kk) {
          const float da = fast_exp2(p.x * Ap[kk]);
          h[kk] = fmaf(da, h[kk], p.y * Bv[kk]);
          ys = fmaf(Cv[kk], h[kk], ys);
        }
        Y[tl][w][lane] = ys;
      }
    };
    if (t0 + T <= L)
      scan_steps(std::true_type{});
    else
      scan_steps(std::false_type{});
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tl = w * TPW + j;
      const int64_t t = t0 + tl;
      if (t < L && dv) {
        float s = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += Y[tl][ww][lane];
        s = fmaf(Dv, keep_u[j], s) * keep_g[j];
        store_io(y, (row0 + t) * D + d, s);
      }
    }
    if (k + 1 < nck) prologue(k + 1);
    __syncthreads();
  }
  if (a.h_final && dv) {
#pragma unroll
    for (int kk = 0; kk < NPL; ++kk) a.h_final[(b * D + d) * N + w * NPL + kk] = h[kk];
  }
}

template <typename IO, int N>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t s) {
  constexpr int NPL = N >= 2 ? 2 : 1;
  constexpr int NW = N / NPL;
  constexpr int T = 16;
  dim3 grid((unsigned)((a.D + 63) / 64), (unsigned)a.B);
  hipLaunchKernelGGL((fwd_chunked_kernel<IO, N, NPL, T>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_fwd_io(const FwdArgs &a, hipStream_t s) {
  switch (a.N) {
    case 1: return launch_fwd_t<IO, 1>(a, s);
    case 2: return launch_fwd_t<IO, 2>(a, s);
    case 4: return launch_fwd_t<IO, 4>(a, s);
    case 8: return launch_fwd_t<IO, 8>(a, s);
    case 16: return launch_fwd_t<IO, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

int64_t fwd_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_fwd(const FwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == 0 ? launch_fwd_io<float>(a, s) : launch_fwd_io<bf16>(a, s);
}

}  // namespace ssm
