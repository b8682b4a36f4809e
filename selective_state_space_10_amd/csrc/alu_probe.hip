// alu_probe.hip -- vector-ALU issue-rate probes for gfx950 (measurement only,
// not part of the scan).  Each kernel runs a fixed count of one instruction
// kind on every lane, in several independent register chains, with one
// workgroup per compute unit (its LDS request leaves room for no second one)
// and W waves per SIMD.  The caller times the launch on its stream with HIP
// events, so the rate follows from wall time, not from a cycle counter.
// Instructions are written in inline asm so that the compiler can neither
// remove nor fuse them; no memory is touched except one store per lane at the
// end (so no load is in flight inside asm).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_alu_probe.h"

namespace {

constexpr int kChains = 8;     // independent dependency chains per lane
constexpr int kGroups = 8;     // unrolled groups per loop iteration
// Dynamic LDS requested at launch (never touched): more than half of a CU's
// LDS, so only one workgroup fits on a CU.
constexpr int kLdsBytes = 96 * 1024;

// KIND 0: v_fma_f32 only.  KIND 1: v_exp_f32 only.  KIND 2: one v_exp_f32
// then four v_fma_f32, each on its own chain (the recurrence's 1:4 mix, no
// instruction waiting for the one before it).  KIND 3: v_mul_f32.  KIND 4: the
// recurrence's own pattern for 8 states of a lane: per state v_mul (step size
// times A), v_exp, v_mul (input times B), the state FMA, and the output FMA
// into one of two running sums.
template <int KIND>
__global__ void probe_kernel(int64_t iters, float *out) {
  float x[kChains], e[kChains];
  const float a = 0.999f + 1e-7f * (float)(threadIdx.x & 7), b = 1e-3f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    x[c] = 0.5f + 0.01f * (float)c + 1e-6f * (float)threadIdx.x;
    e[c] = 0.7f - 0.01f * (float)c;
  }
  float y0 = 0.0f, y1 = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (KIND == 0) {
          asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x[c]) : "v"(a), "v"(b));
        } else if constexpr (KIND == 1) {
          asm volatile("v_exp_f32 %0, -%0" : "+v"(x[c]));  // stays in [0.5, 1]
        } else if constexpr (KIND == 2) {
          // exp on chain c, then FMAs on chains c+1..c+4 (mod 8): consecutive
          // instructions never depend on each other
          asm volatile("v_exp_f32 %0, -%0" : "+v"(e[c]));
          asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x[(c + 1) % kChains]) : "v"(a), "v"(b));
          asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x[(c + 2) % kChains]) : "v"(a), "v"(b));
          asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x[(c + 3) % kChains]) : "v"(a), "v"(b));
          asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x[(c + 4) % kChains]) : "v"(a), "v"(b));
        } else if constexpr (KIND == 3) {
          asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x[c]) : "v"(a));
        } else {
          // state c: arg = dt * A'[c]; da = exp2(arg); in = dtu * B[c];
          // h[c] = da * h[c] + in; y += C[c] * h[c]  (x = h, e = scratch)
          float arg, in;
          asm volatile("v_mul_f32 %0, %1, %2" : "=v"(arg) : "v"(a), "v"(e[c]));
          asm volatile("v_exp_f32 %0, -%0" : "+v"(arg));
          asm volatile("v_mul_f32 %0, %1, %2" : "=v"(in) : "v"(b), "v"(e[c]));
          asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x[c]) : "v"(arg), "v"(in));
          if (c & 1)
            asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(y1) : "v"(e[c]), "v"(x[c]));
          else
            asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(y0) : "v"(e[c]), "v"(x[c]));
        }
      }
    }
  }
  float s = y0 + y1;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c] + e[c];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Which SIMD of its compute unit each wave of a workgroup runs on (the
// SIMD_ID field, bits 5:4, of the HW_ID hardware register), for a workgroup of
// `threads` threads that requests `lds` bytes of LDS.  One value per wave.
__global__ void placement_kernel(int *out) {
  const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);  // hwreg(HW_REG_HW_ID)
  const int wave = threadIdx.x >> 6;
  const int waves = (blockDim.x + 63) >> 6;
  if ((threadIdx.x & 63) == 0) {
    out[(int64_t)blockIdx.x * waves + wave] = (int)((hw >> 4) & 3) | (int)(((hw >> 8) & 15) << 4);
  }
}

}  // namespace

extern "C" {

int ssm_probe_wave_placement(int threads, int lds_bytes, int workgroups, int *out, int64_t out_elems,
                             void *hip_stream) {
  const int waves = (threads + 63) / 64;
  if (threads < 64 || threads > 1024 || lds_bytes < 0 || lds_bytes > 160 * 1024 || workgroups < 1 ||
      out == nullptr || out_elems < (int64_t)workgroups * waves)
    return 1;
  if (hipFuncSetAttribute((const void *)placement_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          lds_bytes) != hipSuccess)
    return 2;
  hipLaunchKernelGGL(placement_kernel, dim3((unsigned)workgroups), dim3((unsigned)threads), lds_bytes,
                     (hipStream_t)hip_stream, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int64_t ssm_probe_instructions_per_lane(int kind, int64_t iters) {
  const int64_t per_group = (kind == 2 || kind == 4) ? 5 : 1;
  return iters * kGroups * kChains * per_group;
}

int ssm_probe_valu(int kind, int waves_per_simd, int64_t iters, float *out, int64_t out_elems,
                   int *workgroups, void *hip_stream) {
  if (kind < 0 || kind > 4 || waves_per_simd < 1 || waves_per_simd > 4 || iters < 1 ||
      out == nullptr || workgroups == nullptr)
    return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 2;
  const int threads = 256 * waves_per_simd;  // 4 SIMDs x W waves x 64 lanes
  if (out_elems < (int64_t)cus * threads) return 1;
  const hipStream_t s = (hipStream_t)hip_stream;
  const dim3 grid((unsigned)cus), block((unsigned)threads);
  // dynamic LDS above 64 KiB must be allowed per kernel
  const void *fns[5] = {(const void *)probe_kernel<0>, (const void *)probe_kernel<1>,
                        (const void *)probe_kernel<2>, (const void *)probe_kernel<3>,
                        (const void *)probe_kernel<4>};
  if (hipFuncSetAttribute(fns[kind], hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess)
    return 2;
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_kernel<0>, grid, block, kLdsBytes, s, iters, out); break;
    case 1: hipLaunchKernelGGL(probe_kernel<1>, grid, block, kLdsBytes, s, iters, out); break;
    case 2: hipLaunchKernelGGL(probe_kernel<2>, grid, block, kLdsBytes, s, iters, out); break;
    case 3: hipLaunchKernelGGL(probe_kernel<3>, grid, block, kLdsBytes, s, iters, out); break;
    default: hipLaunchKernelGGL(probe_kernel<4>, grid, block, kLdsBytes, s, iters, out); break;
  }
  *workgroups = cus;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
