// scan_bwd.hip -- backward of the selective scan for gfx950.
//
// Reverse-mode derivative of the recurrence h_t = exp(dt_t A) h_{t-1} +
// dt_t B_t u_t, y_t = (C_t h_t + D u_t) silu(z_t).  With e_t = dy_t silu(z_t)
// the adjoint of the state runs backwards in time,
//   lambda_t = e_t C_t + exp(dt_{t+1} A) lambda_{t+1}   (lambda_{L} = dh_final),
// and every input gradient is a local product with lambda or e.  States are
// not read from memory: each chunk of kChunkLen steps is recomputed from the
// chunk-boundary state the forward saved (reading guide of arXiv 2312.00752,
// "Donanım Duyarlı Durum Genişletme": intermediate states are recomputed in
// the backward pass).
//
// Mapping: one lane per channel (b, d) holding all N states.  Sums over
// channels (dB, dC) are reduced across the wave and written as per-tile
// partials; sums over batch rows (dA, dD, dbias) as per-row partials; a second
// kernel adds the partials in a fixed order, so results are deterministic.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {

struct BwdWs {
  float *hist;    // (B, ntiles*64, kChunkLen, N): recomputed states of the current chunk
  float *partB;   // (B, ntiles, L, N)
  float *partC;   // (B, ntiles, L, N)
  float *partA;   // (B, D, N)
  float *partD;   // (B, D)
  float *partBias;  // (B, D)
  int64_t ntiles;
};

static inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

static BwdWs carve_ws(void *base, int64_t B, int64_t L, int64_t D, int64_t N, int64_t *total) {
  const int64_t nt = (D + 63) / 64;
  char *p = (char *)base;
  int64_t off = 0;
  BwdWs w;
  w.ntiles = nt;
  auto take = [&](int64_t bytes) {
    float *r = (float *)(p ? p + off : nullptr);
    off += align256(bytes);
    return r;
  };
  w.hist = take(B * nt * 64 * kChunkLen * N * 4);
  w.partB = take(B * nt * L * N * 4);
  w.partC = take(B * nt * L * N * 4);
  w.partA = take(B * D * N * 4);
  w.partD = take(B * D * 4);
  w.partBias = take(B * D * 4);
  if (total) *total = off;
  return w;
}

int64_t bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int) {
  int64_t total = 0;
  carve_ws(nullptr, B, L, D, N, &total);
  return total;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename IO, int N>
__global__ void __launch_bounds__(64) bwd_channel_kernel(BwdArgs a, BwdWs ws) {
  const IO *u = (const IO *)a.u, *dl = (const IO *)a.delta, *zz = (const IO *)a.z;
  const IO *dy = (const IO *)a.dy, *Bm = (const IO *)a.Bm, *Cm = (const IO *)a.Cm;
  const int lane = threadIdx.x;
  const int64_t L = a.L, D = a.D;
  const int64_t b = blockIdx.y, tile = blockIdx.x;
  const int64_t d = tile * 64 + lane;
  const bool dv = d < D;
  const int64_t dc = dv ? d : D - 1;
  const bool sp = a.softplus != 0;
  const float bias = a.bias ? a.bias[dc] : 0.0f;
  const float Dv = a.Dskip ? a.Dskip[dc] : 0.0f;
  const int64_t K = (L + kChunkLen - 1) / kChunkLen;
  float An[N], Ap[N], lam[N], dAacc[N], hst[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    An[n] = a.A[dc * N + n];
    Ap[n] = An[n] * kLog2e;
    lam[n] = (a.dh_final && dv) ? a.dh_final[(b * D + dc) * N + n] : 0.0f;
    dAacc[n] = 0.0f;
  }
  float dD_acc = 0.0f, dbias_acc = 0.0f;
  float *hs = ws.hist + ((b * ws.ntiles * 64 + d) * kChunkLen) * N;

  for (int64_t kc = K - 1; kc >= 0; --kc) {
    const int64_t t0 = kc * kChunkLen;
    const int64_t t1 = (t0 + kChunkLen < L) ? t0 + kChunkLen : L;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      hst[n] = a.chunk_states[((b * K + kc) * D + dc) * N + n];
      h[n] = hst[n];
    }
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t idx = (b * L + t) * D + dc;
      const float dt = step_size(load_io(dl, idx), bias, sp);
      const float dtu = dt * load_io(u, idx);
#pragma unroll
      for (int n = 0; n < N; ++n) {
        h[n] = fmaf(fast_exp2(dt * Ap[n]), h[n], dtu * load_io(Bm, (b * L + t) * N + n));
        hs[(t - t0) * N + n] = h[n];
      }
    }
    for (int64_t t = t1 - 1; t >= t0; --t) {
      const int64_t idx = (b * L + t) * D + dc;
      const int64_t bl = (b * L + t) * N;
      const float s = load_io(dl, idx) + bias;
      const float dt = sp ? softplus_f(s) : s;
      const float x = load_io(u, idx);
      const float dtu = dt * x;
      const float g = load_io(dy, idx);
      const float *ht = hs + (t - t0) * N;
      const float *hp = (t > t0) ? hs + (t - 1 - t0) * N : nullptr;
      float pre = Dv * x;
#pragma unroll
      for (int n = 0; n < N; ++n) pre = fmaf(load_io(Cm, bl + n), ht[n], pre);
      float e = g, dzv = 0.0f;
      if (a.z) {
        const float zv = load_io(zz, idx);
        const float sz = sigmoid_f(zv);
        e = g * zv * sz;
        dzv = g * pre * sz * fmaf(zv, 1.0f - sz, 1.0f);
      }
      if (!dv) e = 0.0f;
      float du_acc = 0.0f, ddt = 0.0f;
      float cB[N], cC[N];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float Bv = load_io(Bm, bl + n), Cv = load_io(Cm, bl + n);
        const float aa = fast_exp2(dt * Ap[n]);
        const float hprev = hp ? hp[n] : hst[n];
        const float lt = fmaf(e, Cv, lam[n]);
        cC[n] = e * ht[n];
        cB[n] = lt * dtu;
        du_acc = fmaf(lt, Bv, du_acc);
        const float r = lt * hprev * aa;
        ddt = fmaf(r, An[n], ddt);
        dAacc[n] = fmaf(r, dt, dAacc[n]);
        lam[n] = aa * lt;
      }
      ddt = fmaf(x, du_acc, ddt);
      const float draw = sp ? ddt * sigmoid_f(s) : ddt;
      if (dv) {
        store_io((IO *)a.du, idx, fmaf(Dv, e, dt * du_acc));
        store_io((IO *)a.ddelta, idx, draw);
        if (a.z) store_io((IO *)a.dz, idx, dzv);
        dbias_acc += draw;
        dD_acc = fmaf(e, x, dD_acc);
      }
      const int64_t po = ((b * ws.ntiles + tile) * L + t) * N;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float vb = wave_sum(cB[n]);
        const float vc = wave_sum(cC[n]);
        if (lane == 0) {
          ws.partB[po + n] = vb;
          ws.partC[po + n] = vc;
        }
      }
    }
  }
  if (dv) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      if (a.dh0) a.dh0[(b * D + d) * N + n] = lam[n];
      ws.partA[(b * D + d) * N + n] = dAacc[n];
    }
    ws.partD[b * D + d] = dD_acc;
    ws.partBias[b * D + d] = dbias_acc;
  }
}

// dB, dC: sum the per-tile partials (fixed tile order), cast to the io type.
template <typename IO>
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(BwdArgs a, BwdWs ws) {
  const int64_t LN = a.L * a.N;
  const int64_t total = a.B * LN;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / LN, r = i % LN;
    float sb = 0.0f, sc = 0.0f;
    for (int64_t tile = 0; tile < ws.ntiles; ++tile) {
      sb += ws.partB[(b * ws.ntiles + tile) * LN + r];
      sc += ws.partC[(b * ws.ntiles + tile) * LN + r];
    }
    store_io((IO *)a.dB, i, sb);
    store_io((IO *)a.dC, i, sc);
  }
}

// dA, dD, dbias: sum the per-row partials over batch rows.
__global__ void __launch_bounds__(256) bwd_reduce_params_kernel(BwdArgs a, BwdWs ws) {
  const int64_t DN = a.D * a.N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < DN) {
    float s = 0.0f;
    for (int64_t b = 0; b < a.B; ++b) s += ws.partA[b * DN + i];
    a.dA[i] = s;
  }
  if (i < a.D) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < a.B; ++b) {
      sd += ws.partD[b * a.D + i];
      sb += ws.partBias[b * a.D + i];
    }
    if (a.dD) a.dD[i] = sd;
    if (a.dbias) a.dbias[i] = sb;
  }
}

template <typename IO, int N>
static hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  BwdWs ws = carve_ws(a.workspace, a.B, a.L, a.D, a.N, nullptr);
  hipLaunchKernelGGL((bwd_channel_kernel<IO, N>), dim3((unsigned)ws.ntiles, (unsigned)a.B), dim3(64), 0, s, a, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = a.B * a.L * a.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((bwd_reduce_bc_kernel<IO>), dim3((unsigned)blocks), dim3(256), 0, s, a, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)((a.D * a.N + 255) / 256)), dim3(256), 0, s, a, ws);
  return hipGetLastError();
}

template <typename IO>
static hipError_t launch_bwd_io(const BwdArgs &a, hipStream_t s) {
  switch (a.N) {
    case 1: return launch_bwd_t<IO, 1>(a, s);
    case 2: return launch_bwd_t<IO, 2>(a, s);
    case 4: return launch_bwd_t<IO, 4>(a, s);
    case 8: return launch_bwd_t<IO, 8>(a, s);
    case 16: return launch_bwd_t<IO, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == 0 ? launch_bwd_io<float>(a, s) : launch_bwd_io<bf16>(a, s);
}

}  // namespace ssm
