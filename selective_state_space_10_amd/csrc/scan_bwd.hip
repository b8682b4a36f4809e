// scan_bwd.hip -- backward of the selective scan for gfx950.
//
// Reverse-mode derivative of the recurrence h_t = exp(dt_t A) h_{t-1} +
// dt_t B_t u_t, y_t = (C_t h_t + D u_t) silu(z_t).  With e_t = dy_t silu(z_t)
// the adjoint of the state runs backwards in time,
//   lambda_t = e_t C_t + exp(dt_{t+1} A) lambda_{t+1}   (from dh_final at the end),
// and every input gradient is a local product with lambda, e or the state.
// States are not read from memory: each chunk of kChunkLen steps is
// recomputed from the chunk-boundary state the forward saved (reading guide
// of arXiv 2312.00752, "Donanım Duyarlı Durum Genişletme": intermediate states
// are recomputed in the backward pass).
//
// One workgroup owns 64 channels (one per lane) of one batch row and all N
// states of them: wave w holds states 2w and 2w+1.  Per chunk of 32 steps:
//   - Prologue (cooperative, 16-byte or 8-byte accesses): dt, dt*u, e, u,
//     d dt/d raw and dy*silu'(z) per (step, channel) into LDS, and B, C.
//   - Recompute: the chunk's states and decay factors, forwards, into
//     registers (32 steps x 2 states x 2 values per lane; with the exact hold
//     or the fused convolution two windows of 16 steps, each recomputed from
//     the chunk start).
//   - Reverse sweep in groups of 8 steps.  Each step leaves three per-lane
//     partial sums over the lane's states in LDS (C h, lambda B, lambda a h A)
//     and the per-state contributions to dB and dC, which are summed over
//     channels: once across lane pairs with a DPP exchange (odd lanes keep
//     their two states in swapped order, so that one add serves both), then
//     through LDS.
//   - Epilogue (one (step, channel) item per thread): sums over the waves,
//     writes du, ddelta and dz, and accumulates dD and d bias.
// Sums over channel tiles (dB, dC) and over batch rows and sequence segments
// (dA, dD, d bias) are written as partials and added by small kernels in a
// fixed order, so results are deterministic.
//
// Long sequences with few channels are split into segments like the forward:
// the adjoint entering a segment from the right is the composition of the
// later segments' affine maps lambda -> exp(A sum dt) lambda + local part.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace ssm {

namespace {

constexpr int kCPW = 64;  // channels per workgroup (one per lane)
constexpr int kTE = 8;    // steps per epilogue group
// recompute windows per chunk (register window of T / windows steps)
template <bool ZOH, bool CONV>
constexpr int kBwdWindows = (ZOH || CONV) ? 2 : 1;
constexpr int kXStride = 36;  // floats per channel-sum staging plane (32 values + padding)
constexpr int kXRot = 12;     // rotation of the odd staging planes
constexpr int kSwap1 = 0xB1;  // DPP quad_perm(1,0,3,2): value of lane ^ 1
constexpr int kSwap2 = 0x4E;  // DPP quad_perm(2,3,0,1): value of lane ^ 2

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

struct BwdWs {
  float *partB, *partC;     // (B, ntiles, L, N): dB, dC summed over one channel tile
  float *partTok;           // (B, ntiles, L): per-token ddelta summed over one channel tile
  float *partA;             // (B, nseg, D, N)
  float *partD, *partBias;  // (B, nseg, D)
  float *lamloc, *carry;    // (B, nseg, D, N): sequence split only
  float *dsum;              // (B, nseg, D)
  float *gconv;             // (B, L, D): gradient at the convolution's pre-activation
  float *cwp, *cbp;         // (B, nrb, D, kMaxConv) and (B, nrb, D): conv tap and bias partials
  int64_t ntiles, nseg, seg_len, nrb;
};

constexpr int64_t kConvRows = 64;  // rows per block of the convolution backward

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Sequence split.  Workgroups (one per CU) run in rounds over the MI355X's
// kCUs compute units, and a partly filled round costs as much as a full one.
// A split into S segments costs R(S x tiles) / S rounds of the full backward
// plus kMode1 of that for the first pass over S - 1 segments (the local
// adjoint carries; measured at 0.23 of a full step), R(w) = ceil(w / kCUs).
// Among the segment counts (1: no split) within 1% of the lowest cost, the
// smallest that gives at least two rounds is taken (later workgroups fill in
// behind the first round's slowest ones: 22.1 ms against 23.5 ms for 32
// against 16 segments at the million-length shape), else the smallest.
// Segments are multiples of 256 steps, at least kMinSeg long: segments this
// short let shapes just above one round fill whole rounds (measured on MI355X:
// the Mamba-2.8b shape, 4 x 4096 x 5120 bf16, 1.97 ms with 2 segments of 2048
// steps against 1.67 ms with 4 of 1024; 10 x 2048 x 2048 fp32 1.04 ms unsplit
// against 0.81 ms with 4 of 512).  Depends on sizes only.
constexpr int64_t kMinSeg = 512;
constexpr int64_t kCUs = 256;
constexpr double kMode1 = 0.23;

int64_t bwd_split_len(int64_t B, int64_t L, int64_t D) {
  const int64_t tiles = B * ((D + kCPW - 1) / kCPW);
  // beyond 16 rounds an unsplit grid wastes at most 1/16 of a round; this
  // also keeps S * tiles far from overflow for any size the API accepts
  if (tiles > 16 * kCUs) return 0;
  const int64_t smax = L / kMinSeg < 1024 ? L / kMinSeg : 1024;
  auto cost = [&](int64_t S) {
    auto rounds = [](int64_t w) { return (double)((w + kCUs - 1) / kCUs); };
    return (rounds(S * tiles) + (S > 1 ? kMode1 * rounds((S - 1) * tiles) : 0.0)) / (double)S;
  };
  double best = cost(1);
  for (int64_t S = 2; S <= smax; ++S) best = cost(S) < best ? cost(S) : best;
  int64_t pick = 0, first = 0;
  for (int64_t S = 1; S <= (smax > 1 ? smax : 1); ++S) {
    if (cost(S) > best * 1.01) continue;
    if (!first) first = S;
    if (S * tiles >= 2 * kCUs) { pick = S; break; }
  }
  if (!pick) pick = first;
  if (pick < 2) return 0;
  int64_t len = (L + pick - 1) / pick;
  len = (len + 255) / 256 * 256;
  return len;
}

BwdWs carve_ws(void *base, int64_t B, int64_t L, int64_t D, int64_t N, int64_t *total, bool conv = false) {
  BwdWs w;
  w.nrb = (L + kConvRows - 1) / kConvRows;
  w.ntiles = (D + kCPW - 1) / kCPW;
  w.seg_len = bwd_split_len(B, L, D);
  w.nseg = w.seg_len ? (L + w.seg_len - 1) / w.seg_len : 1;
  char *p = (char *)base;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    float *r = (float *)(p ? p + off : nullptr);
    off += align256(bytes);
    return r;
  };
  const int64_t S = w.nseg;
  w.partB = take(B * w.ntiles * L * N * 4);
  w.partC = take(B * w.ntiles * L * N * 4);
  w.partTok = take(B * w.ntiles * L * 4);
  w.partA = take(B * S * D * N * 4);
  w.partD = take(B * S * D * 4);
  w.partBias = take(B * S * D * 4);
  if (w.seg_len) {
    w.lamloc = take(B * S * D * N * 4);
    w.carry = take(B * S * D * N * 4);
    w.dsum = take(B * S * D * 4);
  } else {
    w.lamloc = w.carry = w.dsum = nullptr;
  }
  if (conv) {
    w.gconv = take(B * L * D * 4);
    w.cwp = take(B * w.nrb * D * kMaxConv * 4);
    w.cbp = take(B * w.nrb * D * 4);
  } else {
    w.gconv = w.cwp = w.cbp = nullptr;
  }
  if (total) *total = off;
  return w;
}

// MODE 0: full backward of one segment (or of the whole sequence).
// MODE 1: first phase of a sequence split: the adjoint leaving the segment on
// the left from a zero adjoint on the right, and the sum of the step sizes;
// blockIdx.z + 1 is the segment.
// ZOH: the exact zero-order-hold input term coef = expm1(dt A)/A, whose
// derivatives are d coef/d dt = exp(dt A) and d coef/d A = dt^2 psi(dt A).
// CONV: u is recomputed as silu(pre), pre = bias + sum_k w_k x[t - (K-1) + k]
// from the rows of x the convolution reads (loaded with the chunk's other
// inputs), and the gradient is written at the convolution's pre-activation
// (the convolution's own backward runs afterwards).
// Reverse direction and one step size per token are runtime flags; steps are
// numbered in scan order and mapped to memory rows.
template <typename IO, int N, int MODE, bool ZOH, bool CONV>
__global__ void __launch_bounds__(64 * (N >= 2 ? N / 2 : 1)) bwd_kernel(BwdArgs a, BwdWs ws) {
  constexpr int NPL = N >= 2 ? 2 : 1;  // states per lane
  constexpr int NW = N / NPL;          // waves (state slices)
  constexpr int NT = 64 * NW;
  constexpr int CPW = kCPW;
  constexpr int T = (int)kChunkLen;
  constexpr int TE = kTE;
  constexpr int NTG = T / TE;
  static_assert(T % (kBwdWindows<ZOH, CONV> * TE) == 0, "windows must hold whole epilogue groups");
  constexpr int G = CPW / 4;            // 4-channel groups
  constexpr int IPT = T * G / NT;       // prologue items per thread
  constexpr int IPE = TE * CPW / NT;    // epilogue items per thread
  constexpr int BCN = T * N;
  constexpr int BPT = (BCN + NT - 1) / NT;
  static_assert(T % TE == 0 && (T * G) % NT == 0 && IPT >= 1 && (TE * CPW) % NT == 0 && IPE >= 1,
                "work must split evenly over threads");
  static_assert(NT % G == 0, "a thread's channel group must not change between items");
  using V = Vec4<IO>;
  typedef typename V::raw raw_t;

  const IO *__restrict__ u = (const IO *)a.u;
  const IO *__restrict__ dl = (const IO *)a.delta;
  const IO *__restrict__ zz = (const IO *)a.z;
  const IO *__restrict__ dyp = (const IO *)a.dy;
  const IO *__restrict__ Bm = (const IO *)a.Bm;
  const IO *__restrict__ Cm = (const IO *)a.Cm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int par = NPL == 2 ? (lane & 1) : 0;  // odd lanes keep their two states swapped
  const int64_t L = a.L, D = a.D;
  const int64_t tile = blockIdx.x, b = blockIdx.y;
  const int64_t seg = MODE == 1 ? (int64_t)blockIdx.z + 1 : (int64_t)blockIdx.z;
  const int64_t nseg = ws.nseg;
  const int64_t tb = ws.seg_len ? seg * ws.seg_len : 0;
  const int64_t te = ws.seg_len ? (tb + ws.seg_len < L ? tb + ws.seg_len : L) : L;
  const int64_t nck = (te - tb + T - 1) / T;
  const int64_t K = (L + T - 1) / T;
  const int64_t d0 = tile * CPW;
  const int64_t row0 = b * L;
  const bool has_z = a.z != nullptr;
  const bool sp = a.softplus != 0;
  const bool rev = (a.flags & kFlagReverse) != 0;
  const bool tok = (a.flags & kFlagDeltaPerToken) != 0;
  auto mrow = [&](int64_t t) { return rev ? L - 1 - t : t; };  // memory row of scan step t
  constexpr int XK = CONV ? kMaxConv : 1;
  const int ck = CONV ? a.conv_k : 0;
  const IO *__restrict__ xin = (const IO *)a.x;

  __shared__ __attribute__((aligned(16))) float2 P[T][CPW];  // (dt, dt*u), or (dt, u) with ZOH
  __shared__ __attribute__((aligned(16))) float SGC[CONV ? T : 1][CPW];  // silu' at the conv output
  __shared__ __attribute__((aligned(16))) float E[T][CPW];   // dy * silu(z)
  __shared__ __attribute__((aligned(16))) float U[T][CPW];   // u
  __shared__ __attribute__((aligned(16))) float SG[T][CPW];  // d dt / d raw delta
  __shared__ __attribute__((aligned(16))) float GZ[T][CPW];  // dy * silu'(z)
  // B, C of (step, state slice) in the slot order of each lane parity; the
  // second parity's plane is offset by 16 bytes, so that a wave's read of both
  // planes (even and odd lanes) touches different banks
  __shared__ __attribute__((aligned(16))) float BCs[2][T * NW * 4 + 4];
  auto bcs = [&](int pp, int tl, int sl) { return &BCs[pp][(tl * NW + sl) * 4]; };
  __shared__ __attribute__((aligned(16))) float Q[3][TE][NW][64];  // per-lane partials: C h, lambda B, r A
  // Channel-sum staging of dB, dC: 32 values per plane, planes padded to 36
  // floats and odd planes rotated by 12 places, so that both the per-step
  // stores and the channel sums' 16-byte reads are free of bank conflicts.
  __shared__ __attribute__((aligned(16))) float X[NW][TE][4][kXStride];

  // --- prologue ownership: channel group g, steps tl0 + j*(NT/G)
  const int g = tid % G;
  const int tl0 = tid / G;
  const int64_t dg = d0 + 4 * g;
  const bool gv = dg < D;  // D % 4 == 0: a group is all valid or all not
  const int64_t dgc = gv ? dg : D - 4;
  float bias4[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.bias) {
    const float4 v = *(const float4 *)(a.bias + dgc);
    bias4[0] = v.x, bias4[1] = v.y, bias4[2] = v.z, bias4[3] = v.w;
  }
  // convolution taps (zero past the width) and bias per channel, in LDS: read in
  // the prologue only, so they hold no registers through the recurrence
  __shared__ __attribute__((aligned(16))) float CWB[CONV ? CPW : 1][kMaxConv + 1];
  if (CONV) {
    for (int i = tid; i < CPW * (kMaxConv + 1); i += NT) {
      const int c = i / (kMaxConv + 1), kk = i % (kMaxConv + 1);
      const int64_t dd = d0 + c < D ? d0 + c : D - 1;
      float v = 0.0f;
      if (kk < ck)
        v = a.conv_w[dd * ck + kk];
      else if (kk == kMaxConv && a.conv_b)
        v = a.conv_b[dd];
      CWB[c][kk] = v;
    }
    __syncthreads();
  }

  // --- sweep ownership: channel d0 + lane, slot s holds state w*NPL + (s ^ par)
  const int64_t d = d0 + lane;
  const bool dv = d < D;
  const int64_t dc = dv ? d : D - 1;
  const float Dv = (MODE == 0 && a.Dskip) ? a.Dskip[dc] : 0.0f;
  int nst[NPL];
  float Ap[NPL], An[NPL], Ainv[NPL], lam[NPL], dAacc[NPL];
#pragma unroll
  for (int s = 0; s < NPL; ++s) {
    nst[s] = w * NPL + (s ^ par);
    An[s] = a.A[dc * N + nst[s]];
    Ap[s] = An[s] * kLog2e;
    Ainv[s] = ZOH ? 1.0f / An[s] : 0.0f;
    dAacc[s] = 0.0f;
    float l0 = 0.0f;
    if (MODE == 0) {
      if (ws.seg_len)
        l0 = ws.carry[((b * nseg + seg) * D + dc) * N + nst[s]];
      else if (a.dh_final)
        l0 = a.dh_final[(b * D + dc) * N + nst[s]];
    }
    lam[s] = dv ? l0 : 0.0f;
  }
  float dD_acc = 0.0f, dbias_acc = 0.0f, dsum = 0.0f;

  raw_t r_dl[IPT], r_u[IPT], r_z[IPT], r_dy[IPT];
  raw_t r_x[IPT][XK];  // with CONV: the rows of x the convolution reads
  float r_b[BPT], r_c[BPT], r_h[NPL];

  auto load_chunk = [&](int64_t kc) {
    const int64_t t0 = tb + kc * T;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int64_t t = t0 + tl0 + j * (NT / G);
      const int64_t r = row0 + mrow(t < te ? t : te - 1);
      const int64_t idx = r * D + dgc;
      r_dl[j] = tok ? V::splat(dl, r) : V::load(dl, idx);
      r_dy[j] = V::load(dyp, idx);
      if (MODE == 0 && CONV) {  // the rows the causal convolution reads (forward direction only)
        const int64_t tm = t < te ? t : te - 1;
#pragma unroll
        for (int kk = 0; kk < XK; ++kk) {
          const int64_t ts = tm - (ck - 1) + kk;
          r_x[j][kk] = (kk < ck && ts >= 0) ? V::load(xin, (row0 + ts) * D + dgc) : raw_t{};
        }
      } else if (MODE == 0) {
        r_u[j] = V::load(u, idx);
      }
      if (has_z) r_z[j] = V::load(zz, idx);
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = tid + j * NT;
      if (BCN % NT == 0 || i < BCN) {
        const int64_t t = t0 + i / N;
        const int64_t idx = (row0 + mrow(t < te ? t : te - 1)) * N + i % N;
        if (MODE == 0) r_b[j] = load_io(Bm, idx);
        r_c[j] = load_io(Cm, idx);
      }
    }
    if (MODE == 0) {
      const int64_t k = t0 / T;
#pragma unroll
      for (int s = 0; s < NPL; ++s) r_h[s] = a.chunk_states[((b * K + k) * N + nst[s]) * D + dc];
    }
  };

  auto prologue = [&](int64_t kc) {
    const int64_t t0 = tb + kc * T;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const int tl = tl0 + j * (NT / G);
      const bool ok = gv && t0 + tl < te;  // padding steps and channels: dt = 0, e = 0
      const float4 r4 = V::cvt(r_dl[j]), g4 = V::cvt(r_dy[j]);
      float4 x4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (MODE == 0 && CONV) {  // u = silu(pre), pre = bias + sum_k w_k x[t - (K-1) + k]; keep silu'(pre)
        const int cg = 4 * g;
        float pre[4] = {CWB[cg][kMaxConv], CWB[cg + 1][kMaxConv], CWB[cg + 2][kMaxConv], CWB[cg + 3][kMaxConv]};
#pragma unroll
        for (int kk = 0; kk < XK; ++kk) {
          const float4 xv = V::cvt(r_x[j][kk]);
          pre[0] = fmaf(CWB[cg][kk], xv.x, pre[0]);
          pre[1] = fmaf(CWB[cg + 1][kk], xv.y, pre[1]);
          pre[2] = fmaf(CWB[cg + 2][kk], xv.z, pre[2]);
          pre[3] = fmaf(CWB[cg + 3][kk], xv.w, pre[3]);
        }
        float uv[4], sd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sg = sigmoid_f(pre[q]);
          uv[q] = pre[q] * sg;
          sd[q] = sg * fmaf(pre[q], 1.0f - sg, 1.0f);
        }
        x4 = make_float4(uv[0], uv[1], uv[2], uv[3]);
        *(float4 *)&SGC[CONV ? tl : 0][4 * g] = make_float4(sd[0], sd[1], sd[2], sd[3]);
      } else if (MODE == 0) {
        x4 = V::cvt(r_u[j]);
      }
      const float4 z4 = has_z ? V::cvt(r_z[j]) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float rv[4] = {r4.x, r4.y, r4.z, r4.w}, gv4[4] = {g4.x, g4.y, g4.z, g4.w};
      const float xv[4] = {x4.x, x4.y, x4.z, x4.w}, zv[4] = {z4.x, z4.y, z4.z, z4.w};
      float dt[4], e[4], sg[4], gz[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = rv[q] + bias4[q];
        dt[q] = ok ? (sp ? softplus_f(s) : s) : 0.0f;
        sg[q] = sp ? sigmoid_f(s) : 1.0f;
        float ev = gv4[q], gzv = 0.0f;
        if (has_z) {
          const float sz = sigmoid_f(zv[q]);
          ev = gv4[q] * zv[q] * sz;
          gzv = gv4[q] * sz * fmaf(zv[q], 1.0f - sz, 1.0f);
        }
        e[q] = ok ? ev : 0.0f;
        gz[q] = gzv;
      }
      float4 *pp = (float4 *)&P[tl][4 * g];
      if (ZOH) {
        pp[0] = make_float4(dt[0], xv[0], dt[1], xv[1]);
        pp[1] = make_float4(dt[2], xv[2], dt[3], xv[3]);
      } else {
        pp[0] = make_float4(dt[0], dt[0] * xv[0], dt[1], dt[1] * xv[1]);
        pp[1] = make_float4(dt[2], dt[2] * xv[2], dt[3], dt[3] * xv[3]);
      }
      *(float4 *)&E[tl][4 * g] = make_float4(e[0], e[1], e[2], e[3]);
      if (MODE == 0) {
        *(float4 *)&U[tl][4 * g] = x4;
        *(float4 *)&SG[tl][4 * g] = make_float4(sg[0], sg[1], sg[2], sg[3]);
        *(float4 *)&GZ[tl][4 * g] = make_float4(gz[0], gz[1], gz[2], gz[3]);
      }
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int i = tid + j * NT;
      if (BCN % NT == 0 || i < BCN) {
        const int tl = i / N, n = i % N;
        const int sl = n / NPL, k = n % NPL;
        const float bv = MODE == 0 ? r_b[j] : 0.0f;
#pragma unroll
        for (int pp = 0; pp < NPL; ++pp) {
          bcs(pp, tl, sl)[k ^ pp] = bv;
          bcs(pp, tl, sl)[NPL + (k ^ pp)] = r_c[j];
        }
      }
    }
  };

  if (MODE == 1) {
    // Adjoint carry only: lambda <- exp(dt A) (e C + lambda), backwards.
    load_chunk(nck - 1);
    for (int64_t kc = nck - 1; kc >= 0; --kc) {
      prologue(kc);
      if (kc > 0) load_chunk(kc - 1);
      __syncthreads();
#pragma unroll
      for (int tl = T - 1; tl >= 0; --tl) {
        const float dt = P[tl][lane].x;
        const float e = E[tl][lane];
        const float4 bc = *(const float4 *)bcs(par, tl, w);
        const float cv[2] = {NPL == 2 ? bc.z : bc.y, bc.w};
#pragma unroll
        for (int s = 0; s < NPL; ++s) {
          const float lt = fmaf(e, cv[s], lam[s]);
          lam[s] = fast_exp2(dt * Ap[s]) * lt;
        }
        dsum += dt;
      }
      __syncthreads();
    }
    if (dv) {
#pragma unroll
      for (int s = 0; s < NPL; ++s) ws.lamloc[((b * nseg + seg) * D + d) * N + nst[s]] = lam[s];
      if (w == 0) ws.dsum[(b * nseg + seg) * D + d] = dsum;
    }
    return;
  }

  // ---------------------------------------------------------------- MODE 0
  auto epilogue = [&](int64_t kc, int tg) {
    const int64_t t0 = tb + kc * T;
#pragma unroll
    for (int j = 0; j < IPE; ++j) {
      const int tq = (tid + j * NT) / CPW;  // channel of every item is the lane
      const int tl = tg * TE + tq;
      const int64_t t = t0 + tl;
      float ddl = 0.0f;
      if (t < te && dv) {
        float pre = Q[0][tq][0][lane], dua = Q[1][tq][0][lane], dda = Q[2][tq][0][lane];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) {
          pre += Q[0][tq][ww][lane];
          dua += Q[1][tq][ww][lane];
          dda += Q[2][tq][ww][lane];
        }
        const float x = U[tl][lane], e = E[tl][lane], dt = P[tl][lane].x;
        // with ZOH the sweep already folded the input-coefficient terms in
        ddl = (ZOH ? dda : fmaf(x, dua, dda)) * SG[tl][lane];
        const int64_t idx = (row0 + mrow(t)) * D + d;
        const float du = fmaf(Dv, e, ZOH ? dua : dt * dua);
        if (CONV)  // chain through the SiLU; the convolution's backward reads it
          ws.gconv[idx] = du * SGC[CONV ? tl : 0][lane];
        else
          store_io((IO *)a.du, idx, du);
        if (!tok) store_io((IO *)a.ddelta, idx, ddl);
        if (has_z) store_io((IO *)a.dz, idx, GZ[tl][lane] * fmaf(Dv, x, pre));
        dD_acc = fmaf(e, x, dD_acc);
        dbias_acc += ddl;
      }
      if (tok) {  // one step size per token: sum this wave's 64 channels
        const float sdl = wave_sum(ddl);
        if (lane == 0 && t < te) ws.partTok[(b * ws.ntiles + tile) * L + mrow(t)] = sdl;
      }
    }
  };
  // dB, dC over this workgroup's channels: lane (o = lane/2, half = lane%2)
  // adds 16 staged values of output o, then its partner's 16 (the rotation of
  // odd planes only changes which lane of the pair adds which values).
  auto channel_sums = [&](int64_t kc, int tg) {
    const int64_t t0 = tb + kc * T;
    const int o = lane >> 1, half = lane & 1;
    const int tq = o >> 2, q = o & 3;
    const float4 *src = (const float4 *)&X[w][tq][q][16 * half];
    const float4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
    float s = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w)) +
              (((v2.x + v2.y) + (v2.z + v2.w)) + ((v3.x + v3.y) + (v3.z + v3.w)));
    s += dpp_mov<kSwap1>(s);
    if (NPL == 1) s += dpp_mov<kSwap2>(s);  // planes q and q^1 hold the two halves of the lanes
    const int64_t t = t0 + tg * TE + tq;
    if (half == 0 && t < te && (NPL == 2 || (q & 1) == 0)) {
      const int n = NPL == 2 ? w * 2 + (q & 1) : w;
      float *dst = q < 2 ? ws.partB : ws.partC;
      dst[((b * ws.ntiles + tile) * L + mrow(t)) * N + n] = s;
    }
  };

  load_chunk(nck - 1);
  for (int64_t kc = nck - 1; kc >= 0; --kc) {
    prologue(kc);
    float hs[NPL];
#pragma unroll
    for (int s = 0; s < NPL; ++s) hs[s] = r_h[s];
    if (kc > 0) load_chunk(kc - 1);
    __syncthreads();

    if constexpr (kBwdWindows<ZOH, CONV> == 1) {
      // Recompute the chunk's states and decay factors.  With ZOH the decay
      // factors are formed again in the sweep instead: the exact hold's extra
      // terms leave no room for both in registers (they would be spilled).
      float Hh[T][NPL], Ha[ZOH ? 1 : T][NPL];
      {
        float h[NPL];
#pragma unroll
        for (int s = 0; s < NPL; ++s) h[s] = hs[s];
#pragma unroll
        for (int tl = 0; tl < T; ++tl) {
          const float2 p = P[tl][lane];
          const float4 bc = *(const float4 *)bcs(par, tl, w);
          const float bv[2] = {bc.x, bc.y};
#pragma unroll
          for (int s = 0; s < NPL; ++s) {
            const float da = fast_exp2(p.x * Ap[s]);
            const float cf = ZOH ? zoh_coef(p.x, p.x * An[s], da, Ainv[s]) : 1.0f;
            h[s] = fmaf(da, h[s], ZOH ? cf * p.y * bv[s] : p.y * bv[s]);
            Hh[tl][s] = h[s];
            if (!ZOH) Ha[ZOH ? 0 : tl][s] = da;
          }
        }
      }

#pragma unroll
      for (int tg = NTG - 1; tg >= 0; --tg) {
#pragma unroll
        for (int tq = TE - 1; tq >= 0; --tq) {
          const int tl = tg * TE + tq;
          const float2 p = P[tl][lane];
          const float e = E[tl][lane];
          const float4 bc = *(const float4 *)bcs(par, tl, w);
          const float bv[2] = {bc.x, bc.y};
          const float cv[2] = {NPL == 2 ? bc.z : bc.y, bc.w};
          float pre = 0.0f, dup = 0.0f, ddp = 0.0f, cB[NPL], cC[NPL];
#pragma unroll
          for (int s = 0; s < NPL; ++s) {
            const float ht = Hh[tl][s];
            const float hp = tl > 0 ? Hh[tl > 0 ? tl - 1 : 0][s] : hs[s];
            const float lt = fmaf(e, cv[s], lam[s]);
            const float da = ZOH ? fast_exp2(p.x * Ap[s]) : Ha[ZOH ? 0 : tl][s];
            pre = fmaf(cv[s], ht, pre);
            cC[s] = e * ht;
            lam[s] = da * lt;
            const float r = lam[s] * hp;
            ddp = fmaf(r, An[s], ddp);
            dAacc[s] = fmaf(r, p.x, dAacc[s]);
            if (ZOH) {  // p.y is u; the coefficient and its derivatives enter every term
              const float x = p.x * An[s];
              const float cf = zoh_coef(p.x, x, da, Ainv[s]);
              const float lu = lt * p.y;
              cB[s] = lu * cf;
              dup = fmaf(lt * cf, bv[s], dup);
              const float q = lu * bv[s];
              ddp = fmaf(q, da, ddp);
              dAacc[s] = fmaf(q, zoh_dcoef_dA(p.x, x, da, cf, Ainv[s]), dAacc[s]);
            } else {  // p.y is dt*u
              cB[s] = lt * p.y;
              dup = fmaf(lt, bv[s], dup);
            }
          }
          Q[0][tq][w][lane] = pre;
          Q[1][tq][w][lane] = dup;
          Q[2][tq][w][lane] = ddp;
          if constexpr (NPL == 2) {
            const int xi = ((lane >> 1) + kXRot * par) & 31;
            X[w][tq][par][xi] = cB[0] + dpp_mov<kSwap1>(cB[1]);
            X[w][tq][2 + par][xi] = cC[0] + dpp_mov<kSwap1>(cC[1]);
          } else {
            const int xi = ((lane & 31) + kXRot * (lane >> 5)) & 31;
            X[w][tq][lane >> 5][xi] = cB[0];
            X[w][tq][2 + (lane >> 5)][xi] = cC[0];
          }
        }
        __syncthreads();
        epilogue(kc, tg);
        channel_sums(kc, tg);
        __syncthreads();
      }
    } else {
      // The same recompute and sweep in two windows of T/2 steps, the later
      // one first, each recomputed from the chunk start.  A 32-step window
      // spills with the exact hold's or the convolution's extra registers; the
      // extra recompute costs less than the spill (about 3% of the call).  The
      // plain variant keeps the one-window code above: written in this generic
      // form its register allocation gets worse.
      auto run_window = [&](auto window) {
        constexpr int WI = decltype(window)::value;  // window index, later first
        constexpr int TW = T / kBwdWindows<ZOH, CONV>;
        constexpr int T0 = WI * TW;  // first step of the window
        float Hh[TW][NPL], Ha[ZOH ? 1 : TW][NPL], hm[NPL];  // hm: state before step T0
        {
          float h[NPL];
#pragma unroll
          for (int s = 0; s < NPL; ++s) h[s] = hs[s], hm[s] = hs[s];
#pragma unroll
          for (int tl = 0; tl < T0 + TW; ++tl) {
            const float2 p = P[tl][lane];
            const float4 bc = *(const float4 *)bcs(par, tl, w);
            const float bv[2] = {bc.x, bc.y};
#pragma unroll
            for (int s = 0; s < NPL; ++s) {
              const float da = fast_exp2(p.x * Ap[s]);
              const float cf = ZOH ? zoh_coef(p.x, p.x * An[s], da, Ainv[s]) : 1.0f;
              h[s] = fmaf(da, h[s], ZOH ? cf * p.y * bv[s] : p.y * bv[s]);
              if (tl == T0 - 1) hm[s] = h[s];
              if (tl >= T0) {
                Hh[tl >= T0 ? tl - T0 : 0][s] = h[s];
                if (!ZOH) Ha[(ZOH || tl < T0) ? 0 : tl - T0][s] = da;
              }
            }
          }
        }

#pragma unroll
        for (int tg = (T0 + TW) / TE - 1; tg >= T0 / TE; --tg) {
#pragma unroll
          for (int tq = TE - 1; tq >= 0; --tq) {
            const int tl = tg * TE + tq;
            const int ti = tl - T0;  // step within the window
            const float2 p = P[tl][lane];
            const float e = E[tl][lane];
            const float4 bc = *(const float4 *)bcs(par, tl, w);
            const float bv[2] = {bc.x, bc.y};
            const float cv[2] = {NPL == 2 ? bc.z : bc.y, bc.w};
            float pre = 0.0f, dup = 0.0f, ddp = 0.0f, cB[NPL], cC[NPL];
#pragma unroll
            for (int s = 0; s < NPL; ++s) {
              const float ht = Hh[ti][s];
              const float hp = ti > 0 ? Hh[ti > 0 ? ti - 1 : 0][s] : hm[s];
              const float lt = fmaf(e, cv[s], lam[s]);
              const float da = ZOH ? fast_exp2(p.x * Ap[s]) : Ha[ZOH ? 0 : ti][s];
              pre = fmaf(cv[s], ht, pre);
              cC[s] = e * ht;
              lam[s] = da * lt;
              const float r = lam[s] * hp;
              ddp = fmaf(r, An[s], ddp);
              dAacc[s] = fmaf(r, p.x, dAacc[s]);
              if (ZOH) {  // p.y is u; the coefficient and its derivatives enter every term
                const float x = p.x * An[s];
                const float cf = zoh_coef(p.x, x, da, Ainv[s]);
                const float lu = lt * p.y;
                cB[s] = lu * cf;
                dup = fmaf(lt * cf, bv[s], dup);
                const float q = lu * bv[s];
                ddp = fmaf(q, da, ddp);
                dAacc[s] = fmaf(q, zoh_dcoef_dA(p.x, x, da, cf, Ainv[s]), dAacc[s]);
              } else {  // p.y is dt*u
                cB[s] = lt * p.y;
                dup = fmaf(lt, bv[s], dup);
              }
            }
            Q[0][tq][w][lane] = pre;
            Q[1][tq][w][lane] = dup;
            Q[2][tq][w][lane] = ddp;
            if constexpr (NPL == 2) {
              const int xi = ((lane >> 1) + kXRot * par) & 31;
              X[w][tq][par][xi] = cB[0] + dpp_mov<kSwap1>(cB[1]);
              X[w][tq][2 + par][xi] = cC[0] + dpp_mov<kSwap1>(cC[1]);
            } else {
              const int xi = ((lane & 31) + kXRot * (lane >> 5)) & 31;
              X[w][tq][lane >> 5][xi] = cB[0];
              X[w][tq][2 + (lane >> 5)][xi] = cC[0];
            }
          }
          __syncthreads();
          epilogue(kc, tg);
          channel_sums(kc, tg);
          __syncthreads();
        }
      };
      run_window(std::integral_constant<int, 1>{});
      run_window(std::integral_constant<int, 0>{});
    }
  }

  if (dv) {
#pragma unroll
    for (int s = 0; s < NPL; ++s) {
      ws.partA[((b * nseg + seg) * D + d) * N + nst[s]] = dAacc[s];
      if (a.dh0 && seg == 0) a.dh0[(b * D + d) * N + nst[s]] = lam[s];
    }
  }
  // dD and d bias of channel `lane`: one partial per thread, summed over waves.
  Q[0][0][w][lane] = dD_acc;
  Q[1][0][w][lane] = dbias_acc;
  __syncthreads();
  if (w == 0 && dv) {
    float sd = 0.0f, sb = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      sd += Q[0][0][ww][lane];
      sb += Q[1][0][ww][lane];
    }
    ws.partD[(b * nseg + seg) * D + d] = sd;
    ws.partBias[(b * nseg + seg) * D + d] = sb;
  }
}

// Second phase of a sequence split: the adjoint entering every segment from
// the right, carry[S-1] = dh_final, carry[s-1] = exp(A sum dt over s) carry[s]
// + lamloc[s]: a scan of the segments' affine maps from the last segment to
// the first.  One wave per (b, d, n), segments on the lanes in that order (64
// at a time), composed by the wave-wide associative scan.
__global__ void __launch_bounds__(256) bwd_seg_combine_kernel(BwdArgs a, BwdWs ws) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, d, n): uniform over the wave
  if (i >= a.B * a.D * a.N) return;
  const int64_t n = i % a.N, d = (i / a.N) % a.D, b = i / (a.N * a.D);
  const int64_t S = ws.nseg;
  const float Ap = a.A[d * a.N + n] * kLog2e;
  auto slot = [&](int64_t sg) { return ((b * S + sg) * a.D + d) * a.N + n; };
  float carry = a.dh_final ? a.dh_final[i] : 0.0f;
  if (lane == 0) ws.carry[slot(S - 1)] = carry;
  for (int64_t k0 = 0; k0 + 1 < S; k0 += 64) {
    const int64_t k = k0 + lane;
    const bool valid = k + 1 < S;
    const int64_t sg = S - 1 - k;  // the segment whose map this lane holds
    float x = 1.0f, y = 0.0f;      // identity past the first segment
    if (valid) {
      x = fast_exp2(Ap * ws.dsum[(b * S + sg) * a.D + d]);
      y = ws.lamloc[slot(sg)];
    }
    wave_affine_scan(x, y);
    const float c = fmaf(x, carry, y);  // the adjoint leaving segment sg - 1 on the right
    if (valid) ws.carry[slot(sg - 1)] = c;
    carry = __shfl(c, 63, 64);
  }
}

// The same composition for a few segments (at most kFoldMaxSeg): one thread per
// (b, d, n) folds the segments' maps from the last to the first.
constexpr int64_t kFoldMaxSeg = 8;
__global__ void __launch_bounds__(256) bwd_seg_fold_kernel(BwdArgs a, BwdWs ws) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, d, n)
  if (i >= a.B * a.D * a.N) return;
  const int64_t n = i % a.N, d = (i / a.N) % a.D, b = i / (a.N * a.D);
  const int64_t S = ws.nseg;
  const float Ap = a.A[d * a.N + n] * kLog2e;
  auto slot = [&](int64_t sg) { return ((b * S + sg) * a.D + d) * a.N + n; };
  float carry = a.dh_final ? a.dh_final[i] : 0.0f;
  ws.carry[slot(S - 1)] = carry;
  for (int64_t sg = S - 1; sg >= 1; --sg) {  // the adjoint leaving segment sg - 1 on the right
    carry = fmaf(fast_exp2(Ap * ws.dsum[(b * S + sg) * a.D + d]), carry, ws.lamloc[slot(sg)]);
    ws.carry[slot(sg - 1)] = carry;
  }
}

// dB, dC: sum of the per-tile partials in tile order, stored in the io type.
template <typename IO>
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(BwdArgs a, BwdWs ws) {
  const int64_t LN = a.L * a.N;
  const int64_t total = a.B * LN;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / LN, r = i % LN;
    float sb = 0.0f, sc = 0.0f;
    // unrolled so that the loads of several tiles are in flight together; the
    // additions stay in tile order
#pragma unroll 8
    for (int64_t tile = 0; tile < ws.ntiles; ++tile) {
      sb += ws.partB[(b * ws.ntiles + tile) * LN + r];
      sc += ws.partC[(b * ws.ntiles + tile) * LN + r];
    }
    store_io((IO *)a.dB, i, sb);
    store_io((IO *)a.dC, i, sc);
  }
}

// Per-token ddelta: sum of the per-tile partials in tile order.
template <typename IO>
__global__ void __launch_bounds__(256) bwd_reduce_tok_kernel(BwdArgs a, BwdWs ws) {
  const int64_t total = a.B * a.L;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / a.L, r = i % a.L;
    float sd = 0.0f;
#pragma unroll 8
    for (int64_t tile = 0; tile < ws.ntiles; ++tile) sd += ws.partTok[(b * ws.ntiles + tile) * a.L + r];
    store_io((IO *)a.ddelta, i, sd);
  }
}

// Backward of the causal convolution from the gradient g at its pre-activation:
//   dx[b,t,d] = sum_k w[d,k] g[b, t+(K-1)-k, d],
//   dw[d,k] += x[b, t-(K-1)+k, d] g[b,t,d],   dbias[d] += g[b,t,d].
// Taps are padded at the front to width kMaxConv (zero taps), so the windows
// are static.  One thread per (channel, batch row, block of kConvRows rows);
// tap and bias sums are per-block partials.
template <typename IO>
__global__ void __launch_bounds__(256) conv_bwd_kernel(BwdArgs a, BwdWs ws) {
  constexpr int W = kMaxConv;
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = blockIdx.y, rb = blockIdx.z;
  const int64_t L = a.L, D = a.D;
  if (d >= D) return;  // no barrier in this kernel
  const int K = a.conv_k;
  float wp[W];  // padded taps: wp[k'] = w[k' - (W - K)] for k' >= W - K
#pragma unroll
  for (int k = 0; k < W; ++k) wp[k] = k >= W - K ? a.conv_w[d * K + k - (W - K)] : 0.0f;
  const IO *xin = (const IO *)a.x;
  const float *g = ws.gconv;
  const int64_t t0 = rb * kConvRows, t1 = t0 + kConvRows < L ? t0 + kConvRows : L;
  const int64_t base = b * L;
  float gw[W], xw[W];  // gw[j] = g[t + j], xw[k'] = x[t - (W-1) + k']
#pragma unroll
  for (int j = 0; j < W; ++j) {
    gw[j] = t0 + j < L ? g[(base + t0 + j) * D + d] : 0.0f;
    const int64_t ts = t0 - (W - 1) + j;
    xw[j] = ts >= 0 ? load_io(xin, (base + ts) * D + d) : 0.0f;
  }
  float dwp[W] = {0.f, 0.f, 0.f, 0.f}, db = 0.0f;
  for (int64_t t = t0; t < t1; ++t) {
    float dxv = 0.0f;
#pragma unroll
    for (int j = 0; j < W; ++j) dxv = fmaf(wp[W - 1 - j], gw[j], dxv);
    store_io((IO *)a.dx, (base + t) * D + d, dxv);
#pragma unroll
    for (int k = 0; k < W; ++k) dwp[k] = fmaf(xw[k], gw[0], dwp[k]);
    db += gw[0];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) gw[j] = gw[j + 1], xw[j] = xw[j + 1];
    gw[W - 1] = t + W < L ? g[(base + t + W) * D + d] : 0.0f;
    xw[W - 1] = t + 1 < L ? load_io(xin, (base + t + 1) * D + d) : 0.0f;
  }
  const int64_t pi = (b * ws.nrb + rb) * D + d;
#pragma unroll
  for (int k = 0; k < W; ++k) ws.cwp[pi * W + k] = dwp[k];
  ws.cbp[pi] = db;
}

// Convolution taps and bias: sum of the per-block partials in a fixed order.
// Taps and bias of the convolution: sums of the per-(row, block) partials.
// A workgroup covers 64 channels; its 16 waves take every 16th partial row
// each (in increasing order), and the 16 group sums are then added in group
// order, so the result does not depend on timing.
constexpr int kConvRedGroups = 16;
__global__ void __launch_bounds__(64 * kConvRedGroups) conv_reduce_kernel(BwdArgs a, BwdWs ws) {
  constexpr int W = kMaxConv;
  constexpr int NG = kConvRedGroups;
  static_assert(W == 4, "a partial row's taps are one float4");
  __shared__ float S[NG][W + 1][64];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t d = (int64_t)blockIdx.x * 64 + c;
  const bool dv = d < a.D;
  const int64_t dc = dv ? d : a.D - 1;
  const int64_t R = a.B * ws.nrb;
  float sw[W] = {0.f, 0.f, 0.f, 0.f}, sb = 0.0f;
#pragma unroll 4
  for (int64_t r = q; r < R; r += NG) {
    const float4 w4 = *(const float4 *)&ws.cwp[(r * a.D + dc) * W];
    sw[0] += w4.x, sw[1] += w4.y, sw[2] += w4.z, sw[3] += w4.w;
    sb += ws.cbp[r * a.D + dc];
  }
#pragma unroll
  for (int k = 0; k < W; ++k) S[q][k][c] = sw[k];
  S[q][W][c] = sb;
  __syncthreads();
  if (q != 0 || !dv) return;
  float tw[W] = {0.f, 0.f, 0.f, 0.f}, tb = 0.0f;
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int k = 0; k < W; ++k) tw[k] += S[g][k][c];
    tb += S[g][W][c];
  }
  const int K = a.conv_k;
  for (int k = 0; k < K; ++k) a.dconv_w[d * K + k] = tw[k + W - K];
  if (a.dconv_b) a.dconv_b[d] = tb;
}

// dA, dD, d bias: sum of the partials over batch rows and segments.
__global__ void __launch_bounds__(256) bwd_reduce_params_kernel(BwdArgs a, BwdWs ws) {
  const int64_t DN = a.D * a.N;
  const int64_t R = a.B * ws.nseg;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < DN) {
    float s = 0.0f;
#pragma unroll 8
    for (int64_t r = 0; r < R; ++r) s += ws.partA[r * DN + i];
    a.dA[i] = s;
  }
  if (i < a.D) {
    float sd = 0.0f, sb = 0.0f;
#pragma unroll 8
    for (int64_t r = 0; r < R; ++r) {
      sd += ws.partD[r * a.D + i];
      sb += ws.partBias[r * a.D + i];
    }
    if (a.dD) a.dD[i] = sd;
    if (a.dbias) a.dbias[i] = sb;
  }
}

template <typename IO, int N>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  constexpr int NT = 64 * (N >= 2 ? N / 2 : 1);
  const bool conv = a.conv_k > 0;
  BwdWs ws = carve_ws(a.workspace, a.B, a.L, a.D, a.N, nullptr, conv);
  const unsigned tiles = (unsigned)ws.ntiles;
  hipError_t e;
  if (ws.seg_len) {
    hipLaunchKernelGGL((bwd_kernel<IO, N, 1, false, false>), dim3(tiles, (unsigned)a.B, (unsigned)(ws.nseg - 1)), dim3(NT), 0, s,
                       a, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nst = a.B * a.D * a.N;
    if (ws.nseg <= kFoldMaxSeg)
      hipLaunchKernelGGL(bwd_seg_fold_kernel, dim3((unsigned)((nst + 255) / 256)), dim3(256), 0, s, a, ws);
    else
      hipLaunchKernelGGL(bwd_seg_combine_kernel, dim3((unsigned)((nst + 3) / 4)), dim3(256), 0, s, a, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid(tiles, (unsigned)a.B, (unsigned)ws.nseg);
  const bool zoh = (a.flags & kFlagZoh) != 0;
  if (zoh && conv)
    hipLaunchKernelGGL((bwd_kernel<IO, N, 0, true, true>), grid, dim3(NT), 0, s, a, ws);
  else if (zoh)
    hipLaunchKernelGGL((bwd_kernel<IO, N, 0, true, false>), grid, dim3(NT), 0, s, a, ws);
  else if (conv)
    hipLaunchKernelGGL((bwd_kernel<IO, N, 0, false, true>), grid, dim3(NT), 0, s, a, ws);
  else
    hipLaunchKernelGGL((bwd_kernel<IO, N, 0, false, false>), grid, dim3(NT), 0, s, a, ws);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (conv) {
    const unsigned dt = (unsigned)((a.D + 255) / 256);
    hipLaunchKernelGGL((conv_bwd_kernel<IO>), dim3(dt, (unsigned)a.B, (unsigned)ws.nrb), dim3(256), 0, s, a, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(conv_reduce_kernel, dim3((unsigned)((a.D + 63) / 64)), dim3(64 * kConvRedGroups), 0, s, a,
                       ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.flags & kFlagDeltaPerToken) {
    int64_t tb = (a.B * a.L + 255) / 256;
    if (tb > 65536) tb = 65536;
    hipLaunchKernelGGL((bwd_reduce_tok_kernel<IO>), dim3((unsigned)tb), dim3(256), 0, s, a, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t total = a.B * a.L * a.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL((bwd_reduce_bc_kernel<IO>), dim3((unsigned)blocks), dim3(256), 0, s, a, ws);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)((a.D * a.N + 255) / 256)), dim3(256), 0, s, a, ws);
  return hipGetLastError();
}

template <typename IO>
hipError_t launch_bwd_io(const BwdArgs &a, hipStream_t s) {
  switch (a.N) {
    case 1: return launch_bwd_t<IO, 1>(a, s);
    case 2: return launch_bwd_t<IO, 2>(a, s);
    case 4: return launch_bwd_t<IO, 4>(a, s);
    case 8: return launch_bwd_t<IO, 8>(a, s);
    case 16: return launch_bwd_t<IO, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int64_t bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int) {
  int64_t total = 0;
  carve_ws(nullptr, B, L, D, N, &total);
  return total;
}

int64_t bwd_conv_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int) {
  int64_t total = 0;
  carve_ws(nullptr, B, L, D, N, &total, true);
  return total;
}

hipError_t launch_bwd(const BwdArgs &a, int io_dtype, hipStream_t s) {
  return io_dtype == 0 ? launch_bwd_io<float>(a, s) : launch_bwd_io<bf16>(a, s);
}

}  // namespace ssm
