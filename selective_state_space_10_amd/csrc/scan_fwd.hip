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
// Two kernels share this file.
//
// fwd_ws_kernel (16 states, 64-, 80- or 32-channel tiles; every option and both
// passes of a sequence split) specialises waves: recurrence waves only run the
// recurrence (two states per lane); service waves load the inputs a few
// 16-step sub-chunks ahead, stage (dt, dt*u) and B/C in LDS, and sum, gate and
// store the outputs.  A SIMD issues a service wave's plain arithmetic in the
// slots its recurrence waves leave free.
//
// fwd_kernel (1, 2, 4 or 8 states) runs every phase on every wave.
// One workgroup owns CPW consecutive channels of one batch row and walks the
// sequence in chunks of T steps:
//   - Cooperative phases (all threads): every thread owns fixed (step, group of
//     4 channels) items of a chunk and moves them with 16-byte (fp32) or
//     8-byte (bf16) accesses.  The prologue turns (delta, u) into (dt, dt*u)
//     and stores them in LDS once per (t, d); it also stages the chunk's B and
//     C rows in LDS.  The epilogue adds the per-wave partial sums, applies
//     D*u and the SiLU gate, and stores y.
//   - Recurrence (one wave per NPL states): lanes are channels, and each step
//     reads (dt, dt*u) for its lane and the wave's B/C values from LDS,
//     updates the states, and leaves sum_n C h in LDS.
//   - Loads run PD chunks ahead in registers, so that several chunks of
//     input are in flight while the recurrence of the current one executes.
#include <stdlib.h>

#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {

// XCDs of an MI355X (gfx950): workgroups are handed to them in turn.
constexpr int64_t kXcds = 8;

// MODE 0: full forward (y, chunk states, final state).  MODE 1: first phase of
// a sequence split: the segment's (or piece's, as the launcher sets seg_len)
// end state from a zero start, and the sum of its step sizes (no y).
// blockIdx.z is the segment.
// ZOH: exact zero-order-hold input term expm1(dt A)/A * B * u (reading guide,
// "Yöntem", discretisation of B) instead of dt * B * u.  FLAGS: the other
// options (reverse direction, one step size per token, accumulate into y) are
// honoured as runtime flags, with steps numbered in scan order and mapped to
// memory rows; the plain variant (FLAGS false) carries none of that code.
template <typename IO, int N, int NPL, int CPW, int T, int PD, int MODE, bool ZOH, bool FLAGS>
__global__ void __launch_bounds__(64 * N * CPW / (64 * NPL)) fwd_kernel(FwdArgs a) {
  constexpr int NG = 64 / CPW;             // state groups per wave (lanes = CPW channels x NG groups)
  constexpr int NW = N / (NPL * NG);       // waves per workgroup
  constexpr int NT = 64 * NW;              // threads
  constexpr int NSP = N / NPL;             // state slices per channel
  constexpr int G = CPW / 4;               // groups of 4 channels per tile
  constexpr int IPT = T * G / NT;          // (step, channel group) items per thread per chunk
  constexpr int BCN = T * N;               // B (and C) values per chunk
  constexpr int BPT = (BCN + NT - 1) / NT;
  static_assert(NW >= 1 && NSP == NW * NG, "states must split evenly over lanes and waves");
  static_assert((T * G) % NT == 0 && IPT >= 1, "items must split evenly over threads");
  static_assert(kChunkLen % T == 0, "chunk boundaries must fall on chunk starts");
  static_assert(NT % G == 0, "a thread's channel group must not change between items");
  using V = Vec4<IO>;
  typedef typename V::raw raw_t;

  const IO *__restrict__ u = (const IO *)a.u;
  const IO *__restrict__ dl = (const IO *)a.delta;
  const IO *__restrict__ zz = (const IO *)a.z;
  const IO *__restrict__ Bm = (const IO *)a.Bm;
  const IO *__restrict__ Cm = (const IO *)a.Cm;
  IO *__restrict__ y = (IO *)a.y;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t L = a.L, D = a.D;
  const int64_t b = blockIdx.y;
  const int64_t d0 = (int64_t)blockIdx.x * CPW;
  const int64_t row0 = b * L;
  const int64_t seg = blockIdx.z;
  const int64_t nseg = a.seg_len ? (L + a.seg_len - 1) / a.seg_len : 1;  // (phase 1 runs nseg-1 of them)
  const int64_t tb = a.seg_len ? seg * a.seg_len : 0;                           // first step
  const int64_t te = a.seg_len ? (tb + a.seg_len < L ? tb + a.seg_len : L) : L;  // end (exclusive)
  const int64_t nck = (te - tb + T - 1) / T;
  const int64_t K = (L + kChunkLen - 1) / kChunkLen;
  const bool has_z = MODE == 0 && a.z != nullptr;
  const bool sp = a.softplus != 0;
  const bool rev = FLAGS && (a.flags & kFlagReverse) != 0;
  const bool tok = FLAGS && (a.flags & kFlagDeltaPerToken) != 0;
  const bool accum = FLAGS && (a.flags & kFlagAccumulate) != 0;
  const int ck = FLAGS ? a.conv_k : 0;  // width of the causal convolution producing u (0: u given)
  const IO *__restrict__ xin = (const IO *)a.x;
  constexpr int XK = FLAGS ? kMaxConv : 1;
  auto mrow = [&](int64_t t) { return rev ? L - 1 - t : t; };  // memory row of scan step t

  __shared__ __attribute__((aligned(16))) float2 P[T][CPW];  // (dt, dt*u), or (dt, u) with ZOH
  __shared__ __attribute__((aligned(16))) float Y[T][NW][64];       // per-lane partial sum over its states
  __shared__ __attribute__((aligned(16))) float BC[T][NSP][2 * NPL];  // B then C values per state slice

  // --- cooperative-phase ownership: channel group g, steps tl0 + j*(NT/G)
  const int g = tid % G;
  const int tl0 = tid / G;
  const int64_t dg = d0 + 4 * g;
  const bool gv = dg < D;                      // D % 4 == 0: a group is all valid or all not
  const int64_t dgc = gv ? dg : D - 4;
  float bias4[4] = {0.f, 0.f, 0.f, 0.f}, Dsk4[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.bias) {
    const float4 v = *(const float4 *)(a.bias + dgc);
    bias4[0] = v.x, bias4[1] = v.y, bias4[2] = v.z, bias4[3] = v.w;
  }
  if (a.Dskip) {
    const float4 v = *(const float4 *)(a.Dskip + dgc);
    Dsk4[0] = v.x, Dsk4[1] = v.y, Dsk4[2] = v.z, Dsk4[3] = v.w;
  }
  float cw[4][XK], cb4[4] = {0.f, 0.f, 0.f, 0.f};  // convolution taps and bias of the group
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int kk = 0; kk < XK; ++kk) cw[q][kk] = kk < ck ? a.conv_w[(dgc + q) * ck + kk] : 0.0f;
    if (ck && a.conv_b) cb4[q] = a.conv_b[dgc + q];
  }

  // --- recurrence ownership: channel d0 + c, state slice spi = w*NG + gi
  const int c = lane % CPW;
  const int gi = lane / CPW;
  const int spi = w * NG + gi;
  const int64_t d = d0 + c;
  const bool dv = d < D;
  const int64_t dc = dv ? d : D - 1;
  float Ap[NPL], An[NPL], Ainv[NPL], h[NPL];
  float dsum = 0.0f;  // MODE 1: sum of this channel's step sizes over the segment
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int n = spi * NPL + k;
    An[k] = a.A[dc * N + n];
    Ap[k] = An[k] * kLog2e;
    Ainv[k] = ZOH ? 1.0f / An[k] : 0.0f;
    if (MODE == 1)
      h[k] = 0.0f;
    else if (a.seg_len)
      h[k] = a.seg_state[((b * nseg + seg) * D + dc) * N + n];
    else
      h[k] = a.h0 ? a.h0[(b * D + dc) * N + n] : 0.0f;
  }

  raw_t r_raw[PD][IPT], r_u[PD][IPT], r_z[PD][IPT];  // loads in flight
  raw_t r_x[PD][IPT][XK];                              // convolution input rows
  float r_b[PD][BPT], r_c[PD][BPT];
  float4 keep_u[IPT], keep_g[IPT];                     // kept for the epilogue

  auto load_chunk = [&](int64_t k, raw_t(&ra)[IPT], raw_t(&ru)[IPT], raw_t(&rz)[IPT], float(&rb)[BPT],
                        float(&rc)[BPT], raw_t(&rx)[IPT][XK]) {
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int64_t t = tb + k * T + tl0 + j * (NT / G);
      const int64_t r = row0 + mrow(t < te ? t : te - 1);
      const int64_t idx = r * D + dgc;
      ra[j] = tok ? V::splat(dl, r) : V::load(dl, idx);
      if (ck) {  // the rows the causal convolution reads (forward direction only)
        const int64_t tm = t < te ? t : te - 1;
#pragma unroll
        for (int kk = 0; kk < XK; ++kk) {
          const int64_t ts = tm - (ck - 1) + kk;
          rx[j][kk] = (kk < ck && ts >= 0) ? V::load(xin, (row0 + ts) * D + dgc) : raw_t{};
        }
      } else {
        ru[j] = V::load(u, idx);
      }
      if (has_z) rz[j] = V::load(zz, idx);
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = tid + j * NT;
      if (BCN % NT == 0 || i < BCN) {
        const int64_t t = tb + k * T + i / N;
        const int64_t idx = (row0 + mrow(t < te ? t : te - 1)) * N + i % N;
        rb[j] = load_io(Bm, idx);
        if (MODE == 0) rc[j] = load_io(Cm, idx);
      }
    }
  };
  auto prologue = [&](int64_t k, raw_t(&ra)[IPT], raw_t(&ru)[IPT], raw_t(&rz)[IPT], float(&rb)[BPT],
                      float(&rc)[BPT], raw_t(&rx)[IPT][XK]) {
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int tl = tl0 + j * (NT / G);
      const bool tv = tb + k * T + tl < te;  // steps past the end get dt = 0: no state change
      const float4 r = V::cvt(ra[j]);
      float4 x;
      if (ck) {  // u = silu(bias + sum_k w_k x[t - (K-1) + k])
        float pre[4] = {cb4[0], cb4[1], cb4[2], cb4[3]};
#pragma unroll
        for (int kk = 0; kk < XK; ++kk) {
          const float4 xv = V::cvt(rx[j][kk]);
          pre[0] = fmaf(cw[0][kk], xv.x, pre[0]);
          pre[1] = fmaf(cw[1][kk], xv.y, pre[1]);
          pre[2] = fmaf(cw[2][kk], xv.z, pre[2]);
          pre[3] = fmaf(cw[3][kk], xv.w, pre[3]);
        }
        x = make_float4(silu_f(pre[0]), silu_f(pre[1]), silu_f(pre[2]), silu_f(pre[3]));
      } else {
        x = V::cvt(ru[j]);
      }
      const float rv[4] = {r.x, r.y, r.z, r.w}, xv[4] = {x.x, x.y, x.z, x.w};
      float dt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) dt[q] = tv ? step_size(rv[q], bias4[q], sp) : 0.0f;
      float4 *pp = (float4 *)&P[tl][4 * g];
      if (ZOH) {  // the input coefficient depends on the state: keep u itself
        pp[0] = make_float4(dt[0], xv[0], dt[1], xv[1]);
        pp[1] = make_float4(dt[2], xv[2], dt[3], xv[3]);
      } else {
        pp[0] = make_float4(dt[0], dt[0] * xv[0], dt[1], dt[1] * xv[1]);
        pp[1] = make_float4(dt[2], dt[2] * xv[2], dt[3], dt[3] * xv[3]);
      }
      keep_u[j] = x;
      if (has_z) {
        const float4 zv = V::cvt(rz[j]);
        keep_g[j] = make_float4(silu_f(zv.x), silu_f(zv.y), silu_f(zv.z), silu_f(zv.w));
      } else {
        keep_g[j] = make_float4(1.f, 1.f, 1.f, 1.f);
      }
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = tid + j * NT;
      if (BCN % NT == 0 || i < BCN) {
        const int tl = i / N, n = i % N;
        BC[tl][n / NPL][n % NPL] = rb[j];
        BC[tl][n / NPL][NPL + n % NPL] = MODE == 0 ? rc[j] : 0.0f;
      }
    }
  };
  auto epilogue = [&](int64_t k) {
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int tl = tl0 + j * (NT / G);
      const int64_t t = tb + k * T + tl;
      if (t < te && gv) {
        const int64_t yi = (row0 + mrow(t)) * D + dg;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
#pragma unroll
          for (int gg = 0; gg < NG; ++gg) {
            const float4 v = *(const float4 *)&Y[tl][ww][gg * CPW + 4 * g];
            s.x += v.x, s.y += v.y, s.z += v.z, s.w += v.w;
          }
        }
        s.x = fmaf(Dsk4[0], keep_u[j].x, s.x) * keep_g[j].x;
        s.y = fmaf(Dsk4[1], keep_u[j].y, s.y) * keep_g[j].y;
        s.z = fmaf(Dsk4[2], keep_u[j].z, s.z) * keep_g[j].z;
        s.w = fmaf(Dsk4[3], keep_u[j].w, s.w) * keep_g[j].w;
        if (accum) {
          const float4 o = V::cvt(V::load(y, yi));
          s.x += o.x, s.y += o.y, s.z += o.z, s.w += o.w;
        }
        V::store(y, yi, s);
      }
    }
  };
  auto scan_chunk = [&](int64_t k) {
    const int64_t t0 = tb + k * T;
    if (MODE == 0 && a.chunk_states && (t0 % kChunkLen) == 0 && dv) {
      // layout (B, K, N, D): the lanes of a wave write consecutive channels
      float *cs = a.chunk_states + ((b * K + t0 / kChunkLen) * N + spi * NPL) * D + d;
#pragma unroll
      for (int kk = 0; kk < NPL; ++kk) cs[kk * D] = h[kk];
    }
    // LDS reads run one sub-block of SB steps ahead of their use.
    constexpr int SB = 4;
    float2 pv[2][SB];
    float bcv[2][SB][2 * NPL];
    auto read_sub = [&](int j, float2(&pd)[SB], float(&bd)[SB][2 * NPL]) {
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const int tl = j * SB + q;
        pd[q] = P[tl][c];
        if constexpr (NPL == 2) {
          const float4 v = *(const float4 *)&BC[tl][spi][0];
          bd[q][0] = v.x, bd[q][1] = v.y, bd[q][2] = v.z, bd[q][3] = v.w;
        } else {
#pragma unroll
          for (int r = 0; r < 2 * NPL; ++r) bd[q][r] = BC[tl][spi][r];
        }
      }
    };
    read_sub(0, pv[0], bcv[0]);
#pragma unroll
    for (int j = 0; j < T / SB; ++j) {
      if (j + 1 < T / SB) read_sub(j + 1, pv[(j + 1) & 1], bcv[(j + 1) & 1]);
#pragma unroll
      for (int q = 0; q < SB; ++q) {
        const int tl = j * SB + q;
        const float2 p = pv[j & 1][q];
        const float *bc = bcv[j & 1][q];
        float ys = 0.0f;
#pragma unroll
        for (int kk = 0; kk < NPL; ++kk) {
          const float da = fast_exp2(p.x * Ap[kk]);
          if (ZOH) {
            const float cf = zoh_coef(p.x, p.x * An[kk], da, Ainv[kk]);
            h[kk] = fmaf(da, h[kk], cf * p.y * bc[kk]);
          } else {
            h[kk] = fmaf(da, h[kk], p.y * bc[kk]);
          }
          if (MODE == 0) ys = fmaf(bc[NPL + kk], h[kk], ys);
        }
        if (MODE == 0)
          Y[tl][w][lane] = ys;
        else
          dsum += p.x;
      }
    }
  };

  // Prime the pipeline: chunks 0 .. PD-1 in flight, prologue of chunk 0.
#pragma unroll
  for (int s = 0; s < PD; ++s)
    if (s < nck) load_chunk(s, r_raw[s], r_u[s], r_z[s], r_b[s], r_c[s], r_x[s]);
  prologue(0, r_raw[0], r_u[0], r_z[0], r_b[0], r_c[0], r_x[0]);
  __syncthreads();
  // Chunk k uses ring slot k % PD; the loop is unrolled by PD so slots are
  // compile-time register arrays.
  for (int64_t k0 = 0; k0 < nck; k0 += PD) {
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int64_t k = k0 + s;
      if (k < nck) {
        if (k + PD < nck) load_chunk(k + PD, r_raw[s], r_u[s], r_z[s], r_b[s], r_c[s], r_x[s]);
        scan_chunk(k);
        __syncthreads();
        if (MODE == 0) epilogue(k);
        const int sn = (s + 1) % PD;
        if (k + 1 < nck) prologue(k + 1, r_raw[sn], r_u[sn], r_z[sn], r_b[sn], r_c[sn], r_x[sn]);
        __syncthreads();
      }
    }
  }
  if (MODE == 1) {
    if (dv) {
#pragma unroll
      for (int kk = 0; kk < NPL; ++kk) a.seg_hloc[((b * nseg + seg) * D + d) * N + spi * NPL + kk] = h[kk];
      if (spi == 0) a.seg_dsum[(b * nseg + seg) * D + d] = dsum;
    }
  } else if (a.h_final && dv && seg == nseg - 1) {
#pragma unroll
    for (int kk = 0; kk < NPL; ++kk) a.h_final[(b * D + d) * N + spi * NPL + kk] = h[kk];
  }
}

// Forward with wave specialisation: 16 states, tiles of CPW = 64, 80 or 32
// channels of one batch row, optionally one segment of a split sequence.  With
// FLAGS also the reverse direction, one step size per token and accumulation
// into y, with ZOH the exact zero-order hold, with CONV u built by the fused
// causal convolution and SiLU from x (memory order).  MODE 1 is the first pass
// of a sequence split: each segment's (or piece's) end state from a zero start
// and its sum of step sizes, no output.
// The recurrence waves only run the recurrence, two states per lane.  The
// service waves (one per 16 channels) do everything else for the same tile:
// global loads a few sub-chunks ahead, the step-size prologue and B/C staging
// of the next sub-chunk, and the epilogue (sum of the eight partials, D*u,
// gate, store) of the previous one.  A sub-chunk is T steps; LDS buffers
// alternate between sub-chunks, so one barrier per sub-chunk orders
// everything.  On gfx950 plain arithmetic from one wave fills issue slots
// that a recurrence wave on the same SIMD leaves free.
template <typename IO, int CPW, int T, int R, bool FLAGS, int MODE, bool ZOH, bool CONV>
__global__ void __launch_bounds__(64 * (CPW / 8 + CPW / 16)) __attribute__((amdgpu_waves_per_eu(CPW == 32 ? 4 : 1)))
fwd_ws_kernel(FwdArgs a) {
  // Recurrence thread r (of 8 * CPW) holds channel r % CPW of state slice
  // r / CPW; eight slices of 2 states.  CPW = 64: 8 recurrence waves, 4
  // service waves, one workgroup per CU.  CPW = 80: 10 and 5 waves, one
  // workgroup per CU (at most four waves per SIMD, so 128 registers); for
  // channel counts like 5120 whose 64-channel tiles would leave a second,
  // mostly idle round over the CUs.  CPW = 32: 4 and 2 waves, two workgroups
  // per CU (at most four waves per SIMD: with five, the register bound makes
  // the service waves spill and the 2.8b shape runs 17% slower).
  constexpr int N = 16, NRW = CPW / 8, NSV = CPW / 16, NVW = 8, SPL = N / NVW;
  constexpr int G = CPW / 4;                  // 4-channel groups
  constexpr int NV = 64 * NSV;                // service threads
  constexpr int IPT = T * G / NV;             // (step, channel group) items per service thread
  constexpr int BPT = (T * N + NV - 1) / NV;  // B and C values per service thread (the last may repeat one)
  static_assert((CPW == 64 || CPW == 80 || CPW == 32) && SPL % 2 == 0, "B/C in float4 pieces");
  static_assert(IPT >= 1 && IPT * NV == T * G && kChunkLen % T == 0, "sub-chunks tile the chunk");
  using V = Vec4<IO>;
  typedef typename V::raw raw_t;

  const IO *__restrict__ u = (const IO *)a.u;
  const IO *__restrict__ dl = (const IO *)a.delta;
  const IO *__restrict__ zz = (const IO *)a.z;
  const IO *__restrict__ Bm = (const IO *)a.Bm;
  const IO *__restrict__ Cm = (const IO *)a.Cm;
  IO *__restrict__ y = (IO *)a.y;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t L = a.L, D = a.D;
  // Workgroups are handed to the XCDs in turn (workgroup i to XCD i mod 8) and
  // every XCD has its own L2.  Neighbouring tiles share the cache lines at
  // their edges (a row of 80 bf16 channels is 160 bytes), so the (tile, batch
  // row) pairs of an unsplit grid are renumbered to give every XCD one
  // contiguous run of them, and a line shared by two tiles is fetched once.
  int64_t tile = blockIdx.x, b = blockIdx.y;
  if (gridDim.z == 1) {
    const int64_t P = (int64_t)gridDim.x * gridDim.y;
    if (P % kXcds == 0) {
      const int64_t lin = blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
      const int64_t r = (lin % kXcds) * (P / kXcds) + lin / kXcds;
      tile = r % gridDim.x;
      b = r / gridDim.x;
    }
  }
  const int64_t d0 = tile * CPW;
  const int64_t row0 = b * L;
  // With a sequence split, workgroup z scans segment z from its composed
  // start state; steps are counted from the segment's first step tb.
  const int64_t seg = blockIdx.z;
  const int64_t nseg = a.seg_len ? (L + a.seg_len - 1) / a.seg_len : 1;
  const int64_t tb = a.seg_len ? seg * a.seg_len : 0;
  const int64_t Ls = (a.seg_len && tb + a.seg_len < L ? tb + a.seg_len : L) - tb;  // steps in the segment
  const int64_t nck = (Ls + T - 1) / T;  // sub-chunks
  const int64_t K = (L + kChunkLen - 1) / kChunkLen;

  __shared__ __attribute__((aligned(16))) float2 P[2][T][CPW];            // (dt, dt*u), or (dt, u) with ZOH
  __shared__ __attribute__((aligned(16))) float BC[2][T][NVW][2 * SPL];  // B then C per state slice
  __shared__ __attribute__((aligned(16))) float Y[2][T][NVW][CPW];       // per-lane partial sums

  if (w < NRW) {  // ------------------------------------------- recurrence waves
    const int cl = (w * 64 + lane) % CPW;  // channel in the tile
    const int vw = (w * 64 + lane) / CPW;  // state slice: states vw*SPL ..
    const int64_t d = d0 + cl;
    const bool dv = d < D;
    const int64_t dc = dv ? d : D - 1;
    float Ap[SPL], An[SPL], Ainv[SPL], h[SPL], dsum = 0.0f;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int n = vw * SPL + k;
      An[k] = a.A[dc * N + n];
      Ap[k] = An[k] * kLog2e;
      Ainv[k] = ZOH ? 1.0f / An[k] : 0.0f;
      if (MODE == 1)
        h[k] = 0.0f;
      else if (a.seg_len)
        h[k] = a.seg_state[((b * nseg + seg) * D + dc) * N + n];
      else
        h[k] = a.h0 ? a.h0[(b * D + dc) * N + n] : 0.0f;
    }
    __syncthreads();  // sub-chunk 0 staged
    for (int64_t k = 0; k < nck; ++k) {
      const int buf = (int)(k & 1);
      if (MODE == 0 && a.chunk_states && dv && (k * T) % kChunkLen == 0) {  // tb is a multiple of kChunkLen
        float *cs = a.chunk_states + ((b * K + (tb + k * T) / kChunkLen) * N + vw * SPL) * D + d;
#pragma unroll
        for (int kk = 0; kk < SPL; ++kk) cs[kk * D] = h[kk];
      }
#pragma unroll
      for (int tl = 0; tl < T; ++tl) {
        const float2 p = P[buf][tl][cl];
        float bc[2 * SPL];
#pragma unroll
        for (int i = 0; i < SPL / 2; ++i) {
          const float4 q = *(const float4 *)&BC[buf][tl][vw][4 * i];
          bc[4 * i] = q.x, bc[4 * i + 1] = q.y, bc[4 * i + 2] = q.z, bc[4 * i + 3] = q.w;
        }
        float ys = 0.0f;
#pragma unroll
        for (int kk = 0; kk < SPL; ++kk) {
          const float da = fast_exp2(p.x * Ap[kk]);
          if (ZOH) {  // p.y is u: the input coefficient expm1(dt A)/A depends on the state
            const float cf = zoh_coef(p.x, p.x * An[kk], da, Ainv[kk]);
            h[kk] = fmaf(da, h[kk], cf * p.y * bc[kk]);
          } else {
            h[kk] = fmaf(da, h[kk], p.y * bc[kk]);
          }
          if (MODE == 0) ys = fmaf(bc[SPL + kk], h[kk], ys);
        }
        if (MODE == 0)
          Y[buf][tl][vw][cl] = ys;
        else
          dsum += p.x;
      }
      __syncthreads();
    }
    if (MODE == 1) {
      if (dv) {
#pragma unroll
        for (int kk = 0; kk < SPL; ++kk) a.seg_hloc[((b * nseg + seg) * D + d) * N + vw * SPL + kk] = h[kk];
        if (vw == 0) a.seg_dsum[(b * nseg + seg) * D + d] = dsum;
      }
    } else if (a.h_final && dv && tb + Ls == L) {
#pragma unroll
      for (int kk = 0; kk < SPL; ++kk) a.h_final[(b * D + d) * N + vw * SPL + kk] = h[kk];
    }
    return;  // the service waves' last epilogue needs no further barrier
  }

  // ---------------------------------------------------------------- service waves
  const int vt = tid - NRW * 64;
  const int g = vt % G;
  const int tl0 = vt / G;  // items: steps tl0 + j * (NV / G)
  const int64_t dg = d0 + 4 * g;
  const bool gv = dg < D;  // D % 4 == 0: a group is all valid or all not
  const int64_t dgc = gv ? dg : D - 4;
  const bool has_z = a.z != nullptr;
  const IO *__restrict__ xin = (const IO *)a.x;
  const IO *__restrict__ zsrc = has_z ? zz : CONV ? xin : u;  // loaded either way: no register slot is conditional
  constexpr int XK = CONV ? kMaxConv : 1;
  const int ck = CONV ? a.conv_k : 0;
  const bool sp = a.softplus != 0;
  const bool rev = FLAGS && (a.flags & kFlagReverse) != 0;
  const bool tok = FLAGS && (a.flags & kFlagDeltaPerToken) != 0;
  const bool accum = FLAGS && (a.flags & kFlagAccumulate) != 0;
  auto mrow = [&](int64_t t) {  // memory row of segment step t
    return row0 + (rev ? L - 1 - (tb + t) : tb + t);
  };
  // Addresses: 32-bit byte offsets from the segment's first row in memory (a
  // uniform base), advanced by one sub-chunk per iteration and clamped to the
  // segment's rows by one med3 (steps past the end read the last step).  The
  // launcher keeps (segment length + 64) rows of a (B,L,D) array below 2^31
  // bytes.
  constexpr int SZ = (int)sizeof(IO);
  const int64_t lo = rev ? row0 + L - tb - Ls : row0 + tb;  // lowest memory row of the segment
  const int DS = (int)D * SZ, NS = N * SZ;                   // bytes per row: (B,L,D) and (B,L,N) arrays
  const int kstep = (rev ? -T : T) * DS, kstep_bc = (rev ? -T : T) * NS, kstep_tok = (rev ? -T : T) * SZ;
  const char *__restrict__ u_b = (const char *)(u + lo * D);
  const char *__restrict__ dl_b = (const char *)(dl + lo * D);
  const char *__restrict__ dlt_b = (const char *)(dl + lo);  // one step size per token: (B,L)
  const char *__restrict__ B_b = (const char *)(Bm + lo * N);
  const char *__restrict__ C_b = (const char *)(Cm + lo * N);
  const char *__restrict__ z_b = (const char *)(zsrc + lo * D);
  char *__restrict__ y_b = (char *)(y + lo * D);
  auto seg_row = [&](int t) { return rev ? (int)Ls - 1 - t : t; };  // row of sub-chunk-0 step t from lo
  int o_it[IPT], o_tok[IPT], o_bc[BPT];  // offsets at sub-chunk 0, before clamping
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    o_it[j] = seg_row(tl0 + j * (NV / G)) * DS + (int)dgc * SZ;
    o_tok[j] = seg_row(tl0 + j * (NV / G)) * SZ;
  }
  const int it_lo = (int)dgc * SZ, it_hi = ((int)Ls - 1) * DS + (int)dgc * SZ, tok_hi = ((int)Ls - 1) * SZ;
  int bc_lo[BPT], bc_hi[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int i = BPT * NV > T * N ? (vt + j * NV) % (T * N) : vt + j * NV;  // past T*N: a repeat, not staged
    o_bc[j] = seg_row(i / N) * NS + (i % N) * SZ;
    bc_lo[j] = (i % N) * SZ;
    bc_hi[j] = ((int)Ls - 1) * NS + (i % N) * SZ;
  }
  auto clampi = [](int v, int lo_, int hi_) { return min(max(v, lo_), hi_); };  // one v_med3_i32
  float bias4[4] = {0.f, 0.f, 0.f, 0.f}, Dsk4[4] = {0.f, 0.f, 0.f, 0.f};
  float cw[4][XK], cb4[4] = {0.f, 0.f, 0.f, 0.f};  // convolution taps (zero past the width) and bias
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int kk = 0; kk < XK; ++kk) cw[q][kk] = CONV && kk < ck ? a.conv_w[(dgc + q) * ck + kk] : 0.0f;
    if (CONV && a.conv_b) cb4[q] = a.conv_b[dgc + q];
  }
  if (a.bias) {
    const float4 v = *(const float4 *)(a.bias + dgc);
    bias4[0] = v.x, bias4[1] = v.y, bias4[2] = v.z, bias4[3] = v.w;
  }
  if (a.Dskip) {
    const float4 v = *(const float4 *)(a.Dskip + dgc);
    Dsk4[0] = v.x, Dsk4[1] = v.y, Dsk4[2] = v.z, Dsk4[3] = v.w;
  }

  raw_t r_dl[R][IPT], r_u[R][IPT], r_z[R][IPT];  // loads in flight: sub-chunk j in slot j % R
  raw_t r_x[R][IPT][XK];                          // with CONV: the rows of x the convolution reads
  float r_b[R][BPT], r_c[R][BPT];
  float4 keep_du[2][IPT], keep_g[2][IPT];         // D*u and silu(z), by sub-chunk parity

  // Loads of sub-chunk k; `zero` (always 0) only orders them after its producer.
  auto load_chunk = [&](int64_t k, int zero, raw_t(&ra)[IPT], raw_t(&ru)[IPT], raw_t(&rz)[IPT], float(&rb)[BPT],
                        float(&rc)[BPT], raw_t(&rx)[IPT][XK]) {
    const int kk32 = (int)k;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t o = (uint32_t)clampi(o_it[j] + zero + kk32 * kstep, it_lo, it_hi);
      if (FLAGS && tok)
        ra[j] = V::splat_b(dlt_b, (uint32_t)clampi(o_tok[j] + zero + kk32 * kstep_tok, 0, tok_hi));
      else
        ra[j] = V::load_b(dl_b, o);
      if (CONV) {  // rows r-(K-1) .. r, clamped into the sequence (rows before 0 are zeroed later)
        const int64_t t = k * T + tl0 + j * (NV / G) + zero;
        const int64_t r = mrow(t < Ls ? t : Ls - 1);
#pragma unroll
        for (int kk = 0; kk < XK; ++kk) {
          int64_t ts = r - row0 - (ck - 1) + kk;
          ts = ts < 0 ? 0 : ts < L ? ts : L - 1;
          rx[j][kk] = V::load(xin, (row0 + ts) * D + dgc);
        }
      } else {
        ru[j] = V::load_b(u_b, o);
      }
      if (MODE == 0) rz[j] = V::load_b(z_b, o);
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const uint32_t o = (uint32_t)clampi(o_bc[j] + zero + kk32 * kstep_bc, bc_lo[j], bc_hi[j]);
      rb[j] = load_io_b<IO>(B_b, o);
      if (MODE == 0) rc[j] = load_io_b<IO>(C_b, o);
    }
  };
  auto prologue = [&](int64_t k, raw_t(&ra)[IPT], raw_t(&ru)[IPT], raw_t(&rz)[IPT], float(&rb)[BPT],
                      float(&rc)[BPT], raw_t(&rx)[IPT][XK], float4(&kdu)[IPT], float4(&kg)[IPT]) {
    const int buf = (int)(k & 1);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int tl = tl0 + j * (NV / G);
      const bool tv = (int)k * T + tl < (int)Ls;  // steps past the end get dt = 0: no state change
      const float4 r = V::cvt(ra[j]);
      float4 x;
      if (CONV) {  // u = silu(bias + sum_k w_k x[t - (K-1) + k]), x = 0 before the first row
        const int64_t tm = tb + (k * T + tl < Ls ? k * T + tl : Ls - 1);
        float pre[4] = {cb4[0], cb4[1], cb4[2], cb4[3]};
#pragma unroll
        for (int kk = 0; kk < XK; ++kk) {
          const bool inb = tm - (ck - 1) + kk >= 0;
          const float4 xr = V::cvt(rx[j][kk]);
          const float4 xv = inb ? xr : make_float4(0.f, 0.f, 0.f, 0.f);
          pre[0] = fmaf(cw[0][kk], xv.x, pre[0]);
          pre[1] = fmaf(cw[1][kk], xv.y, pre[1]);
          pre[2] = fmaf(cw[2][kk], xv.z, pre[2]);
          pre[3] = fmaf(cw[3][kk], xv.w, pre[3]);
        }
        x = make_float4(silu_f(pre[0]), silu_f(pre[1]), silu_f(pre[2]), silu_f(pre[3]));
      } else {
        x = V::cvt(ru[j]);
      }
      const float rv[4] = {r.x, r.y, r.z, r.w}, xv[4] = {x.x, x.y, x.z, x.w};
      float dt[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = rv[q] + bias4[q];
        const float sv = softplus_f(s);
        dt[q] = tv ? (sp ? sv : s) : 0.0f;
      }
      float4 *pp = (float4 *)&P[buf][tl][4 * g];
      if (ZOH) {
        pp[0] = make_float4(dt[0], xv[0], dt[1], xv[1]);
        pp[1] = make_float4(dt[2], xv[2], dt[3], xv[3]);
      } else {
        pp[0] = make_float4(dt[0], dt[0] * xv[0], dt[1], dt[1] * xv[1]);
        pp[1] = make_float4(dt[2], dt[2] * xv[2], dt[3], dt[3] * xv[3]);
      }
      // D*u now rather than in the epilogue: a product, unlike u itself, is a
      // new value, so the raw slot can be refilled without a register copy
      // that would wait for the refill's loads.
      if (MODE == 1) continue;
      kdu[j] = make_float4(Dsk4[0] * x.x, Dsk4[1] * x.y, Dsk4[2] * x.z, Dsk4[3] * x.w);
      if (has_z) {
        const float4 zv = V::cvt(rz[j]);
        kg[j] = make_float4(silu_f(zv.x), silu_f(zv.y), silu_f(zv.z), silu_f(zv.w));
      } else {
        kg[j] = make_float4(1.f, 1.f, 1.f, 1.f);
      }
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = vt + j * NV;
      if (BPT * NV > T * N && i >= T * N) continue;
      const int tl = i / N, n = i % N;
      BC[buf][tl][n / SPL][n % SPL] = rb[j];
      if (MODE == 0) BC[buf][tl][n / SPL][SPL + n % SPL] = rc[j];
    }
  };
  auto epilogue = [&](int64_t k, const float4(&kdu)[IPT], const float4(&kg)[IPT]) {
    const int buf = (int)(k & 1);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int tl = tl0 + j * (NV / G);
      if ((int)k * T + tl < (int)Ls && gv) {
        float4 s = *(const float4 *)&Y[buf][tl][0][4 * g];
#pragma unroll
        for (int ww = 1; ww < NVW; ++ww) {
          const float4 v = *(const float4 *)&Y[buf][tl][ww][4 * g];
          s.x += v.x, s.y += v.y, s.z += v.z, s.w += v.w;
        }
        s.x = (s.x + kdu[j].x) * kg[j].x;
        s.y = (s.y + kdu[j].y) * kg[j].y;
        s.z = (s.z + kdu[j].z) * kg[j].z;
        s.w = (s.w + kdu[j].w) * kg[j].w;
        const uint32_t yo = (uint32_t)(o_it[j] + (int)k * kstep);  // t < Ls: no clamp
        if (accum) {
          const float4 o = V::cvt(V::load_b(y_b, yo));
          s.x += o.x, s.y += o.y, s.z += o.z, s.w += o.w;
        }
        V::store_b(y_b, yo, s);
      }
    }
  };

  // Loads and prologues of sub-chunks past the end are harmless (rows are
  // clamped, steps past L get dt = 0, and nothing reads them), so they run
  // unconditionally: a register slot that is only sometimes refilled would
  // make the compiler copy it and wait for loads still in flight.
#pragma unroll
  for (int j = 0; j < R; ++j) load_chunk(j, 0, r_dl[j], r_u[j], r_z[j], r_b[j], r_c[j], r_x[j]);
  prologue(0, r_dl[0], r_u[0], r_z[0], r_b[0], r_c[0], r_x[0], keep_du[0], keep_g[0]);
  load_chunk(R, 0, r_dl[0], r_u[0], r_z[0], r_b[0], r_c[0], r_x[0]);
  __syncthreads();  // sub-chunk 0 staged
  // Iteration k (the recurrence waves scan sub-chunk k): epilogue of k-1,
  // then prologue of k+1 and the loads of k+1+R into the slot it frees.
  // The loop is unrolled so that every slot index is a constant.
  constexpr int U = R % 2 ? 2 * R : R;
  auto iteration = [&](int64_t k, const int i) {  // i = k % U
    const int rs = (i + 1) % R, ks = (i + 1) % 2;  // slots of sub-chunk k+1 (and k-1 for ks)
    if (MODE == 0 && k >= 1) epilogue(k - 1, keep_du[ks], keep_g[ks]);
    prologue(k + 1, r_dl[rs], r_u[rs], r_z[rs], r_b[rs], r_c[rs], r_x[rs], keep_du[ks], keep_g[ks]);
    // The refill must follow the slot's last use: hoisted above it, it would
    // need other registers and a copy at the loop edge that waits for it.
    // The zero below is produced only after every value of the slot and every
    // product of the prologue (so none of them is computed later from the
    // slot), and the refill's addresses depend on it.
    int zero = MODE == 0 ? after_all(0, keep_du[ks], keep_g[ks], r_z[rs], r_c[rs]) : 0;
    if constexpr (CONV)
      zero = after_all(zero, r_dl[rs], r_x[rs], r_b[rs]);
    else
      zero = after_all(zero, r_dl[rs], r_u[rs], r_b[rs]);
    load_chunk(k + 1 + R, zero, r_dl[rs], r_u[rs], r_z[rs], r_b[rs], r_c[rs], r_x[rs]);
    __syncthreads();
  };
  int64_t k = 0;
  for (; k + U <= nck; k += U) {
#pragma unroll
    for (int i = 0; i < U; ++i) iteration(k + i, i);
  }
#pragma unroll
  for (int i = 0; i < U - 1; ++i)
    if (k + i < nck) iteration(k + i, i);
  if (MODE == 1) return;
  if ((nck - 1) & 1)
    epilogue(nck - 1, keep_du[1], keep_g[1]);
  else
    epilogue(nck - 1, keep_du[0], keep_g[0]);
}

// Wave-specialised forward configuration.  Measured on MI355X at 8 x 2048 x
// 2048 x 16 (fp32): eight recurrence waves (two per SIMD, 2 states per lane)
// with 16-step sub-chunks beat four (one per SIMD) with 32-step ones, and a
// ring of two register slots beats four (which spills).
constexpr int kWsSteps = 16, kWsRing = 2;

// Launches the wave-specialised forward variant for the arguments' options.
template <typename IO, int CPW, int MODE, bool ZOH>
static void launch_ws(const FwdArgs &a, dim3 grid, hipStream_t s) {
  const dim3 block(64 * (CPW / 8 + CPW / 16));
  if (a.conv_k) {
    hipLaunchKernelGGL((fwd_ws_kernel<IO, CPW, kWsSteps, kWsRing, true, MODE, ZOH, true>), grid, block, 0, s, a);
    return;
  }
  if (a.flags)
    hipLaunchKernelGGL((fwd_ws_kernel<IO, CPW, kWsSteps, kWsRing, true, MODE, ZOH, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((fwd_ws_kernel<IO, CPW, kWsSteps, kWsRing, false, MODE, ZOH, false>), grid, block, 0, s, a);
}

// Second phase of a sequence split: the state entering every segment,
// h_in[0] = h0, h_in[s+1] = exp(A * sum of dt over s) * h_in[s] + h_loc[s],
// i.e. an exclusive scan of the segments' affine maps.  The first pass may have
// cut each segment into `pieces` pieces: then the maps composed are the
// pieces' ((nseg - 1) * pieces of them; their end states and step-size sums
// have rows of nrow pieces), and the state after every pieces-th one is the
// start state of a segment.  One wave per (b, d, n), pieces on the lanes (64
// at a time), composed by the wave-wide associative scan; the state is carried
// from one group of 64 to the next.
__global__ void __launch_bounds__(256) fwd_seg_combine_kernel(FwdArgs a, int64_t nseg, int64_t pieces,
                                                               int64_t nrow) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, d, n): uniform over the wave
  if (i >= a.B * a.D * a.N) return;
  const int64_t n = i % a.N, d = (i / a.N) % a.D, b = i / (a.N * a.D);
  const float Ap = a.A[d * a.N + n] * kLog2e;
  auto slot = [&](int64_t sg) { return ((b * nseg + sg) * a.D + d) * a.N + n; };   // segment starts
  auto pslot = [&](int64_t pc) { return ((b * nrow + pc) * a.D + d) * a.N + n; };  // piece end states
  const int64_t nmap = (nseg - 1) * pieces;
  float carry = a.h0 ? a.h0[i] : 0.0f;
  if (lane == 0) a.seg_state[slot(0)] = carry;
  for (int64_t s0 = 0; s0 < nmap; s0 += 64) {
    const int64_t pc = s0 + lane;  // the piece whose map this lane holds
    const bool valid = pc < nmap;
    float x = 1.0f, y = 0.0f;      // identity past the last map
    if (valid) {
      x = fast_exp2(Ap * a.seg_dsum[(b * nrow + pc) * a.D + d]);
      y = a.seg_hloc[pslot(pc)];
    }
    wave_affine_scan(x, y);
    const float h = fmaf(x, carry, y);  // the state after piece pc
    if (valid && (pc + 1) % pieces == 0) a.seg_state[slot((pc + 1) / pieces)] = h;
    carry = __shfl(h, 63, 64);
  }
}

// The same composition for a few maps (at most kFoldMaxSeg): one thread per
// (b, d, n) folds the pieces' maps in order, h <- exp(A sum dt_p) h + hloc_p,
// so that no wave spends most of its lanes on absent maps (accesses are
// coalesced along d and n).
constexpr int64_t kFoldMaxSeg = 8;
__global__ void __launch_bounds__(256) fwd_seg_fold_kernel(FwdArgs a, int64_t nseg, int64_t pieces,
                                                            int64_t nrow) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, d, n)
  if (i >= a.B * a.D * a.N) return;
  const int64_t n = i % a.N, d = (i / a.N) % a.D, b = i / (a.N * a.D);
  const float Ap = a.A[d * a.N + n] * kLog2e;
  auto slot = [&](int64_t sg) { return ((b * nseg + sg) * a.D + d) * a.N + n; };
  auto pslot = [&](int64_t pc) { return ((b * nrow + pc) * a.D + d) * a.N + n; };
  float h = a.h0 ? a.h0[i] : 0.0f;
  a.seg_state[slot(0)] = h;
  const int64_t nmap = (nseg - 1) * pieces;
  for (int64_t pc = 0; pc < nmap; ++pc) {
    h = fmaf(fast_exp2(Ap * a.seg_dsum[(b * nrow + pc) * a.D + d]), h, a.seg_hloc[pslot(pc)]);
    if ((pc + 1) % pieces == 0) a.seg_state[slot((pc + 1) / pieces)] = h;
  }
}

// Sequence split for problems with too few channel tiles to fill the GPU:
// segments of at least kMinSeg steps.  With 16 states both passes run the
// wave-specialised kernel on 64-channel tiles, one workgroup per CU, in rounds
// over kSplitCUs (the CUs of an MI355X); a partly filled round costs as much as
// a full one.  S segments cost R(S x tiles) / S rounds of the full pass plus
// kSplitMode1 of that for the first pass over S - 1 segments (measured: 0.78
// of a full step), R(w) = ceil(w / kSplitCUs).  Among the counts within 1% of
// the lowest cost the smallest giving at least kSplitMinRounds rounds is taken
// (later workgroups fill in behind earlier ones: at the million-length shape
// 7.9 ms with one round of 16 segments, 7.3 with two, 7.2 with four), else
// the smallest.  Other state counts aim at kSplitTarget workgroups of 32
// channels.  Depends on sizes only, so the workspace query agrees with it.
constexpr int64_t kMinSeg = 4096;
constexpr int64_t kSplitTarget = 512;
constexpr int64_t kSplitCUs = 256;
constexpr double kSplitMode1 = 0.78;
constexpr int64_t kSplitMinRounds = 4;

// The wave-specialised kernel addresses a segment with 32-bit byte offsets:
// (segment length + 64) rows of a (B,L,D) array must stay below 2^31 bytes.
static int64_t ws_max_rows(int64_t D, int64_t io_bytes) { return ((int64_t)1 << 31) / (D * io_bytes) - 64; }

// Segment length of a sequence split (0: no split), io_bytes per element.
static int64_t split_len(int64_t B, int64_t L, int64_t D, int64_t N, int64_t io_bytes) {
  const int64_t tiles64 = B * ((D + 63) / 64);
  if (tiles64 >= 128 || L < 2 * kMinSeg) return 0;
  const int64_t tiles32 = B * ((D + 31) / 32);
  int64_t nseg = (kSplitTarget + tiles32 - 1) / tiles32;
  if (N == 16) {
    const int64_t smax = L / kMinSeg < 1024 ? L / kMinSeg : 1024;
    auto cost = [&](int64_t S) {
      auto rounds = [](int64_t w) { return (double)((w + kSplitCUs - 1) / kSplitCUs); };
      return (rounds(S * tiles64) + (S > 1 ? kSplitMode1 * rounds((S - 1) * tiles64) : 0.0)) / (double)S;
    };
    double best = cost(1);
    for (int64_t S = 2; S <= smax; ++S) best = cost(S) < best ? cost(S) : best;
    int64_t pick = 0, first = 0;
    for (int64_t S = 1; S <= (smax > 1 ? smax : 1); ++S) {
      if (cost(S) > best * 1.01) continue;
      if (!first) first = S;
      if (S * tiles64 >= kSplitMinRounds * kSplitCUs) {
        pick = S;
        break;
      }
    }
    nseg = pick ? pick : first;
  }
  if (nseg > L / kMinSeg) nseg = L / kMinSeg;
  if (nseg < 2) return 0;
  int64_t len = (L + nseg - 1) / nseg;
  len = (len + kChunkLen - 1) / kChunkLen * kChunkLen;
  // more, shorter segments where a segment would not fit 32-bit offsets
  // (D < 8192 here, so the cap is at least 65472 steps)
  const int64_t cap = ws_max_rows(D, io_bytes) / kChunkLen * kChunkLen;
  return len < cap ? len : cap;
}

// Steps per piece of a split's first pass (16 states).  The first pass runs on
// the S - 1 segments before the last, and with few channel tiles it leaves CUs
// idle (at the 32K-context shape 2 x 80 workgroups on 256 CUs).  Cut into k
// pieces of len / k steps (a multiple of kChunkLen, at least kMinPiece), it
// runs R((S - 1) k tiles) rounds of pieces k times shorter; the smallest k with
// the fewest such rounds per unit of length is taken if that saves at least 5%
// (k = 1 where no cut helps, as at the million-length shape).  Pieces are kept
// long enough that a workgroup's start (its first loads in flight) stays a
// small part of its time.  Depends on sizes only.
constexpr int64_t kMinPiece = 2048;
static int64_t piece_len(int64_t B, int64_t L, int64_t D, int64_t N, int64_t io_bytes) {
  const int64_t len = split_len(B, L, D, N, io_bytes);
  if (len == 0 || N != 16) return len;
  const int64_t nseg = (L + len - 1) / len;
  const int64_t first = (nseg - 1) * B * ((D + 63) / 64);  // first-pass workgroups, uncut
  auto rounds = [](int64_t w) { return (double)((w + kSplitCUs - 1) / kSplitCUs); };
  int64_t best_k = 1;
  double best = rounds(first);
  for (int64_t k = 2; len / k >= kMinPiece && k <= 64; ++k) {
    if (len % (k * kChunkLen) != 0) continue;
    const double c = rounds(k * first) / (double)k;
    if (c < best * 0.95) best = c, best_k = k;
  }
  return len / best_k;
}

// Channels per workgroup (CPW) for dstate N.  A 64-channel tile takes a CU
// (84 KB of LDS), an 80-channel one too (104 KB); 32-channel tiles fit two
// (16 states) or three (fwd_kernel) per CU.  Measured on MI355X: 64-channel
// tiles are fastest while the grid fits in one round over the CUs; beyond
// that, 16 states take the width with the fewest costed rounds (pick_cpw),
// other state counts take 32-channel tiles.  SSM_FWD_CPW overrides the choice
// (tuning only).
static int device_cus() {
  static int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return 256;
    return n;
  }();
  return cus;
}

template <int N>
static int pick_cpw(const FwdArgs &a, int64_t io_bytes) {
  static const int env = [] {
    const char *e = getenv("SSM_FWD_CPW");
    return e ? atoi(e) : 0;
  }();
  constexpr int NPL = N >= 2 ? 2 : 1;
  constexpr int mincpw = 64 * NPL / N > 16 ? 64 * NPL / N : 16;
  if (env == 16 || env == 32 || env == 64 || (N == 16 && env == 80)) return env < mincpw ? mincpw : env;
  if (mincpw > 32) return 64;
  if (split_len(a.B, a.L, a.D, a.N, 4)) return 32;  // split sequences use 32-channel tiles (the io size only caps the length)
  const int64_t cus = device_cus();
  const int64_t wg64 = a.B * ((a.D + 63) / 64);
  if (wg64 <= cus) return 64;
  if constexpr (N == 16) {
    // More tiles than one round of 64 channels: the width with the lowest
    // cost in rounds.  A partly filled round costs as much as a full one.  A
    // round of 64- or 80-channel tiles (one workgroup per CU) costs its width;
    // a CU holding two 32-channel workgroups costs 83 and one alone 35
    // (measured on MI355X: 16 x 2048 x 2048 fp32 takes 331 us on 64-channel
    // tiles, 372 on 80, 400 on 32; 12 x 2048 x 2048 takes 285 on 32, 289 on
    // 64; 8 x 4096 x 5120 bf16 takes 710 on 80, 795 on 64, 905 on 32).  With
    // the fused convolution in fp32 the 80- and 32-channel variants spill
    // registers (their x rows in flight are 16-byte values): a round of 80
    // costs 102 (4 x 4096 x 5120: 0.557 ms on 80 in one round, 0.693 ms on 64
    // in two), and 32-channel tiles are never the fastest (1.10 ms there;
    // 12 x 2048 x 2040: 0.58 ms on 32, 0.38 on 64).  In bf16 the costs above
    // hold with the convolution too.
    auto rounds = [&](int64_t wg) { return (wg + cus - 1) / cus; };
    const bool conv_f32 = a.conv_k != 0 && io_bytes == 4;
    const int64_t wg32 = a.B * ((a.D + 31) / 32);
    const int64_t full = wg32 / (2 * cus), rest = wg32 % (2 * cus);
    const int64_t c32 = conv_f32 ? INT64_MAX : full * 83 + (rest == 0 ? 0 : rest > cus ? 83 : 35);
    const int64_t c64 = rounds(wg64) * 64;
    const int64_t c80 = rounds(a.B * ((a.D + 79) / 80)) * (conv_f32 ? 102 : 80);
    if (c64 <= c80 && c64 <= c32) return 64;
    return c80 <= c32 ? 80 : 32;
  }
  return 32;
}

template <typename IO, int N, int CPW, bool ZOH, bool FLAGS>
static hipError_t launch_fwd_cpw(const FwdArgs &a0, hipStream_t s) {
  constexpr int NPL = N >= 2 ? 2 : 1;
  constexpr int NW = N * CPW / (64 * NPL);
  constexpr int T = 32;
  constexpr int IPT = T * (CPW / 4) / (64 * NW);
  constexpr int PD = IPT <= 2 ? 2 : 1;
  FwdArgs a = a0;
  a.seg_len = split_len(a.B, a.L, a.D, a.N, sizeof(IO));
  const unsigned tiles = (unsigned)((a.D + CPW - 1) / CPW);
  if (a.seg_len == 0) {
    hipLaunchKernelGGL((fwd_kernel<IO, N, NPL, CPW, T, PD, 0, ZOH, FLAGS>), dim3(tiles, (unsigned)a.B, 1), dim3(64 * NW), 0, s,
                       a);
    return hipGetLastError();
  }
  const int64_t nseg = (a.L + a.seg_len - 1) / a.seg_len;
  // the first pass's pieces: pieces per segment, and rows of pieces over the
  // whole length (the layout of their end states and step-size sums)
  const int64_t plen = piece_len(a.B, a.L, a.D, a.N, sizeof(IO));
  const int64_t pieces = a.seg_len / plen, nrow = (a.L + plen - 1) / plen;
  float *ws = (float *)a.workspace;
  a.seg_hloc = ws;
  a.seg_state = ws + a.B * nrow * a.D * a.N;
  a.seg_dsum = a.seg_state + a.B * nseg * a.D * a.N;
  // 16 states: both passes run the wave-specialised kernel on 64-channel tiles
  constexpr bool kWs = N == 16;
  const unsigned t64 = (unsigned)((a.D + 63) / 64);
  if constexpr (kWs) {
    FwdArgs a1 = a;  // the first pass over pieces of plen steps
    a1.seg_len = plen;
    launch_ws<IO, 64, 1, ZOH>(a1, dim3(t64, (unsigned)a.B, (unsigned)((nseg - 1) * pieces)), s);
  } else {
    hipLaunchKernelGGL((fwd_kernel<IO, N, NPL, CPW, T, PD, 1, ZOH, FLAGS>), dim3(tiles, (unsigned)a.B, (unsigned)(nseg - 1)),
                       dim3(64 * NW), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nst = a.B * a.D * a.N;
  if ((nseg - 1) * pieces <= kFoldMaxSeg)
    hipLaunchKernelGGL(fwd_seg_fold_kernel, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, s, a, nseg, pieces, nrow);
  else
    hipLaunchKernelGGL(fwd_seg_combine_kernel, dim3((unsigned)((nst + 3) / 4)), dim3(256), 0, s, a, nseg, pieces,
                       nrow);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (kWs) {  // the segments' full scans
    launch_ws<IO, 64, 0, ZOH>(a, dim3(t64, (unsigned)a.B, (unsigned)nseg), s);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd_kernel<IO, N, NPL, CPW, T, PD, 0, ZOH, FLAGS>), dim3(tiles, (unsigned)a.B, (unsigned)nseg),
                     dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// The launch plan of a forward call: which kernel, how many channels per
// workgroup, and the sequence split.  The launcher follows it and
// ssm_scan_fwd_plan reports it, so the two cannot disagree.
template <int N>
static FwdPlan plan_fwd_t(const FwdArgs &a, int64_t io_bytes) {
  constexpr int NPL = N >= 2 ? 2 : 1;
  constexpr int mincpw = 64 * NPL / N > 16 ? 64 * NPL / N : 16;
  // options use one tile width (fewer instantiations); the plain scan picks its own
  constexpr int OCPW = mincpw > 32 ? 64 : 32;
  FwdPlan pl{};
  pl.segment_len = split_len(a.B, a.L, a.D, a.N, io_bytes);
  pl.segments = pl.segment_len ? (a.L + pl.segment_len - 1) / pl.segment_len : 1;
  pl.first_pass_len = piece_len(a.B, a.L, a.D, a.N, io_bytes);
  if (N == 16 && pl.segment_len == 0 && a.L <= ws_max_rows(a.D, io_bytes)) {
    // 16 states, no sequence split, and every row of a (B,L,D) array within
    // 32-bit offsets: the wave-specialised kernel, also for the options
    pl.kernel = kPlanWaveSpecialised;
    int cpw = pick_cpw<N>(a, io_bytes);
    if (cpw == 16) cpw = 32;              // (a tuning override; 32 is the narrowest tile here)
    pl.tile_channels = cpw;
    return pl;
  }
  int cpw;
  if (a.flags || a.conv_k) {
    cpw = OCPW;
  } else {
    const int c = pick_cpw<N>(a, io_bytes);
    cpw = (mincpw <= 16 && c == 16) ? 16 : (mincpw <= 32 && c == 32) ? 32 : 64;
  }
  if (N == 16 && pl.segment_len) {  // both passes of a split: the wave-specialised kernel, 64-channel tiles
    pl.kernel = kPlanWaveSpecialised;
    pl.tile_channels = 64;
  } else {
    pl.kernel = kPlanAllPurpose;
    pl.tile_channels = cpw;
  }
  return pl;
}

static FwdPlan plan_fwd_n(const FwdArgs &a, int64_t io_bytes) {
  switch (a.N) {
    case 1: return plan_fwd_t<1>(a, io_bytes);
    case 2: return plan_fwd_t<2>(a, io_bytes);
    case 4: return plan_fwd_t<4>(a, io_bytes);
    case 8: return plan_fwd_t<8>(a, io_bytes);
    default: return plan_fwd_t<16>(a, io_bytes);
  }
}

FwdPlan plan_fwd(const FwdArgs &a, int io_dtype) { return plan_fwd_n(a, io_dtype == 0 ? 4 : 2); }

template <typename IO, int N>
static hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t s) {
  const FwdPlan pl = plan_fwd_t<N>(a, sizeof(IO));
  const bool zoh = (a.flags & kFlagZoh) != 0;
  if constexpr (N == 16) {
    if (pl.kernel == kPlanWaveSpecialised && pl.segments == 1) {
      const int cpw = pl.tile_channels;
      const dim3 grid((unsigned)((a.D + cpw - 1) / cpw), (unsigned)a.B, 1);
      if (cpw == 64) {
        zoh ? launch_ws<IO, 64, 0, true>(a, grid, s) : launch_ws<IO, 64, 0, false>(a, grid, s);
      } else if (cpw == 80) {
        zoh ? launch_ws<IO, 80, 0, true>(a, grid, s) : launch_ws<IO, 80, 0, false>(a, grid, s);
      } else {  // 32-channel tiles: several workgroups per CU
        zoh ? launch_ws<IO, 32, 0, true>(a, grid, s) : launch_ws<IO, 32, 0, false>(a, grid, s);
      }
      return hipGetLastError();
    }
  }
  // the all-purpose kernel, or a split sequence (launch_fwd_cpw runs both passes)
  constexpr int NPL = N >= 2 ? 2 : 1;
  constexpr int mincpw = 64 * NPL / N > 16 ? 64 * NPL / N : 16;
  constexpr int OCPW = mincpw > 32 ? 64 : 32;
  if (zoh) return launch_fwd_cpw<IO, N, OCPW, true, true>(a, s);
  if (a.flags || a.conv_k) return launch_fwd_cpw<IO, N, OCPW, false, true>(a, s);
  if constexpr (mincpw <= 16) {
    if (pl.tile_channels == 16) return launch_fwd_cpw<IO, N, 16, false, false>(a, s);
  }
  if constexpr (mincpw <= 32) {
    if (pl.tile_channels == 32) return launch_fwd_cpw<IO, N, 32, false, false>(a, s);
  }
  return launch_fwd_cpw<IO, N, 64, false, false>(a, s);
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

// Scratch memory of the allocation-free forward (ssm_scan_fwd_noalloc): the
// sequence split's per-segment states and step-size sums live here instead of
// in a caller workspace.  One copy per device, held while the code object is
// loaded; every call on a device shares it.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): it
// asks the runtime for the device address once per device, below.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null until looked up)
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {  // first call on this device, which is current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int64_t fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int io_dtype) {
  const int64_t io_bytes = io_dtype == 0 ? 4 : 2;
  const int64_t len = split_len(B, L, D, N, io_bytes);
  if (len == 0) return 0;
  const int64_t nseg = (L + len - 1) / len;
  const int64_t nrow = (L + piece_len(B, L, D, N, io_bytes) - 1) / piece_len(B, L, D, N, io_bytes);
  // end states and step-size sums of the first pass's pieces; segment start states
  return (B * nrow * D * N + B * nrow * D + B * nseg * D * N) * 4;
}

hipError_t launch_fwd(const FwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == 0 ? launch_fwd_io<float>(a, s) : launch_fwd_io<bf16>(a, s);
}

}  // namespace ssm
