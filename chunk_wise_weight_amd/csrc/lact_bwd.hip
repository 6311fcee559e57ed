// Backward of the LaCT SwiGLU fast-weight layer for gfx950 (review of "Test-Time
// Training Done Right", LaCT Model Architecture §1, eq. (3)-(4), differentiated by
// the chain rule; the squared error summed over each chunk, plain GD).
//
// The states W_c (the operand copies each chunk's update starts from) are first
// recomputed by the forward kernels, keys only, and kept.  Then, from the last
// chunk back, with g the fp32 gradient with respect to the state after chunk c
// (zero after the last one):
//   queries (applied with W_{c+1}, or with W_c in apply-then-update order):
//     Aq = Q W1^T, Uq = Q W3^T, Hq = silu(Aq) Uq, dHq = dO W2,
//     dAq = dHq Uq silu'(Aq), dUq = dHq silu(Aq),
//     g2 += dO^T Hq, g1 += dAq^T Q, g3 += dUq^T Q, dq = dAq W1 + dUq W3;
//   the update W_{c+1} = W_c - eta G(W_c; k, v), with upstream gG = -eta g:
//     A = k W1^T, U = k W3^T, S = silu(A), Hh = S U, R = Hh W2^T - v,
//     dH = R W2, dA = dH U silu'(A), dU = dH S            (the forward's gradient)
//     ddA = k gG1^T, ddU = k gG3^T,
//     ddH = ddA U silu'(A) + ddU S,
//     dR = Hh gG2^T + ddH W2^T,  dv = -dR,
//     dHh = R gG2 + dR W2,
//     dU_f = ddA dH silu'(A) + dHh S,
//     dA_f = ddA dH U silu''(A) + (ddU dH + dHh U) silu'(A),
//     dk = dA gG1 + dU gG3 + dA_f W1 + dU_f W3,
//     g2 += R^T ddH + dR^T Hh, g1 += dA_f^T k, g3 += dU_f^T k
//   (silu'(a) = s(1 + a(1 - s)), silu''(a) = s(1 - s)(2 + a(1 - 2s)), s the
//   logistic function).  Finally the initial weights' gradients are g summed over
//   the batch rows of each head.
//
// Every contraction is one launch of a batched engine GEMM over the (batch, head)
// rows: out[q][p] = alpha sum_k Q[q][k] P[p][k] over one or two K streams, each
// operand K-major or MN-major (a token-major matrix read with the tokens as K).
// Elementwise passes between them form the gate terms.  Layouts as in the
// forward: q, k, v, dO [BH, n, dh]; per-chunk intermediates [BH, C, m] or
// [BH, C, dh]; states and gradients [BH, 3, m dh] (W1 [m, dh], W3 [m, dh],
// W2 [dh, m]).
#include <type_traits>

#include "gemm.hpp"
#include "launch.hpp"

namespace ttt {

namespace {

template <typename T> constexpr int bsz() { return (int)sizeof(T); }
inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// One operand of a batched GEMM: element (r, k) of batch b at base + b bs + r ld + k
// (K-major) or base + b bs + k ld + r (MN-major); ld and bs in elements.
struct BOp {
  const void* base;
  int64_t ld, bs;
};

// Output modes.  The gate modes finish an elementwise stage in the epilogue
// from the tile's fp32 values x and inputs in[] read at the same positions
// (layout of out), with s the logistic of A, S = silu(A) = A s and
// silu'(A) = s (1 + A (1 - s)):
//   kGateKey: out = dH = x;  eo0 = dA = x U silu'(A), eo1 = dU = x S
//             (in: A, U)
//   kGateQ:   x = dHq (not stored);  eo0 = dAq = x U silu'(A), eo1 = dUq = x S
//             (in: Aq, Uq)
//   kGateF:   x = dHh (not stored);  eo0 = dA_f = ddA dH U silu''(A) + (ddU dH +
//             x U) silu'(A), eo1 = dU_f = ddA dH silu'(A) + x S
//             (in: A, U, dH, ddA, ddU)
//   kStoreNeg: out = x and eo0 = -x (eo0 rows ldo apart, batch stride eo_so)
enum { kStoreT = 0, kStoreF32 = 1, kAccF32 = 2, kGateKey = 4, kGateQ = 5, kGateF = 6, kStoreNeg = 7 };

struct BGemm {
  BOp P[4], Q[4];
  int K[4];          // contraction length of each stream (0: the stream is empty)
  int NP, NQ, batch;
  void* out;         // out[b][q][p] at out + b so + q ldo + p
  int64_t ldo, so;
  float alpha;
  const void* in[5];  // the gate modes' inputs (dtype, layout of out)
  void* eo[2];        // the gate modes' and kStoreNeg's extra outputs (dtype)
  int64_t eo_so;      // kStoreNeg: batch stride of eo[0]
};

// Up to three GEMMs of one kind in one launch (their tiles one after the
// other), each contraction split nsplit ways along K: split s covers K steps
// [s ks, (s + 1) ks) of every stream and writes out + b so + s split_so.
constexpr int kMaxSet = 3;
struct BGemmSet {
  BGemm g[kMaxSet];
  int n, nsplit;
  int64_t split_so;
};

template <typename T, bool MN, int ROWS>
using OpOf = std::conditional_t<MN, DmaOpMN<T, Wide::NW, ROWS>, DmaOp<Wide::NW, ROWS>>;

template <typename T, bool MN, int ROWS>
__device__ __forceinline__ void init_op(OpOf<T, MN, ROWS>& op, const BOp& o, int b, int r0, int nrows, int K,
                                        int k0 = 0) {
  const T* base = (const T*)o.base + (int64_t)b * o.bs + (MN ? (int64_t)k0 * o.ld : (int64_t)k0);
  if constexpr (MN)
    op.init(base + r0, min(ROWS, nrows - r0), (uint64_t)o.ld * bsz<T>(), K);
  else
    op.init(base + (int64_t)r0 * o.ld, nullptr, min(ROWS, nrows - r0), (uint64_t)o.ld * bsz<T>(),
            (unsigned)((uint64_t)K * bsz<T>()));
}

// Batched GEMM on the engine's 256 x 256 tile; PMN / QMN pick the operand
// layouts (shared by both streams), NS the number of K streams, MODE the output.
template <typename T, bool PMN, bool QMN, int NS, int MODE>
TTT_GEMM_KERNEL(Wide) void k_bgemm(BGemmSet set) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  constexpr int KR = 128 / bsz<T>();
  // which GEMM of the set: the workgroups of g[0] first, then g[1], then g[2],
  // in dispatch order, so that a set listing its longest tiles first starts
  // them in the first round; the XCD-aware order then applies within each GEMM
  int id = blockIdx.x, which = 0;
#pragma unroll
  for (int i = 0; i < kMaxSet - 1; ++i) {
    const BGemm& gi = set.g[i];
    const int tiles = ((gi.NP + G::BP - 1) / G::BP) * ((gi.NQ + G::BQ - 1) / G::BQ) * gi.batch * set.nsplit;
    if (which == i && i + 1 < set.n && id >= tiles) {
      id -= tiles;
      which = i + 1;
    }
  }
  const BGemm& g = set.g[which];
  const int TP = (g.NP + G::BP - 1) / G::BP, TQ = (g.NQ + G::BQ - 1) / G::BQ, per = TP * TQ;
  id = xcd_remap(id, per * g.batch * set.nsplit);
  const int bs_ = id / per;
  const int b = bs_ / set.nsplit, sp = bs_ - b * set.nsplit;
  int tp, tq;
  grouped_tile(id - bs_ * per, TP, TQ, 4, tp, tq);
  const int p0 = tp * G::BP, q0 = tq * G::BQ;
  // this split's K range, whole K steps (every stream the same)
  int kmax = 0;
#pragma unroll
  for (int st = 0; st < NS; ++st) kmax = max(kmax, g.K[st]);
  const int ks = ((kmax + set.nsplit - 1) / set.nsplit + KR - 1) / KR * KR;
  const int k0 = sp * ks;
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  // the streams one after the other on one accumulator, each with its own
  // operand state, so that only one stream's DMA offsets are live at a time
  // (two at once spill); each K loop ends on a barrier, so the next may refill
  // the stages at once
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const int Ks = max(0, min(ks, g.K[st] - k0));
    if (Ks <= 0) continue;
    OpOf<T, PMN, G::BP> op;
    OpOf<T, QMN, G::BQ> oq;
    init_op<T, PMN, G::BP>(op, g.P[st], b, p0, g.NP, Ks, k0);
    init_op<T, QMN, G::BQ>(oq, g.Q[st], b, q0, g.NQ, Ks, k0);
    mainloop<T, G>(op, oq, (Ks + KR - 1) / KR, acc, smem, NoHook{});
  }

  // out[q][p]: staged by rows q (p contiguous), in passes when a whole tile
  // does not fit the stage area
  using TO = std::conditional_t<MODE == kStoreF32 || MODE == kAccF32, float, T>;
  constexpr bool GATE = MODE == kGateKey || MODE == kGateQ || MODE == kGateF;
  constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(float) + G::Smem - 1) / G::Smem, RPP = G::BQ / PASSES;
  const Staged<float, G::BP> st{smem};
  const int qn = min(G::BQ, g.NQ - q0), pn = min(G::BP, g.NP - p0);
  TO* out = (TO*)g.out + (int64_t)b * g.so + (int64_t)sp * set.split_so;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int jq = 0; jq < G::NQB; ++jq) {
      const int qq = G::acc_q(jq) - ps * RPP;
      if (qq < 0 || qq >= RPP) continue;
#pragma unroll
      for (int ib = 0; ib < G::NPB; ++ib)
        st.put4(qq, G::acc_p(ib, 0), g.alpha * acc[ib][jq][0], g.alpha * acc[ib][jq][1], g.alpha * acc[ib][jq][2],
                g.alpha * acc[ib][jq][3]);
    }
    __syncthreads();
    const int rows = max(0, min(RPP, qn - ps * RPP));
    if constexpr (GATE) {
      // 8-element spans (16-byte reads of bf16 inputs); the gate modes' outputs are [C, m] tiles, m % 8 == 0
      constexpr int SPANS = G::BP / 8;
      for (int idx = threadIdx.x; idx < rows * SPANS; idx += G::NT) {
        const int r = idx / SPANS, c = (idx - r * SPANS) * 8;
        if (c >= pn) continue;
        const int64_t o = (int64_t)(q0 + ps * RPP + r) * g.ldo + p0 + c;
        const int64_t e = (int64_t)b * g.so + o;
        float x[8], A[8], U[8], dH[8], ddA[8], ddU[8], y0[8], y1[8];
        {
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(smem + st.off(r, c));
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(smem + st.off(r, c + 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = v0[i];
            x[4 + i] = v1[i];
          }
        }
        auto in8 = [&](int i, float* d) {
          const T* p = (const T*)g.in[i] + e;
          const f32x4 a0 = load4(p), a1 = load4(p + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            d[j] = a0[j];
            d[4 + j] = a1[j];
          }
        };
        in8(0, A);
        in8(1, U);
        if constexpr (MODE == kGateF) {
          in8(2, dH);
          in8(3, ddA);
          in8(4, ddU);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sg = sigmoid_f(A[i]), S = A[i] * sg, s1 = sg * (1.0f + A[i] * (1.0f - sg));
          if constexpr (MODE == kGateF) {
            const float s2 = sg * (1.0f - sg) * (2.0f + A[i] * (1.0f - 2.0f * sg));
            y0[i] = ddA[i] * dH[i] * U[i] * s2 + (ddU[i] * dH[i] + x[i] * U[i]) * s1;
            y1[i] = ddA[i] * dH[i] * s1 + x[i] * S;
          } else {
            y0[i] = x[i] * U[i] * s1;
            y1[i] = x[i] * S;
          }
        }
        T* e0 = (T*)g.eo[0] + e;
        T* e1 = (T*)g.eo[1] + e;
        store4(e0, y0[0], y0[1], y0[2], y0[3]);
        store4(e0 + 4, y0[4], y0[5], y0[6], y0[7]);
        store4(e1, y1[0], y1[1], y1[2], y1[3]);
        store4(e1 + 4, y1[4], y1[5], y1[6], y1[7]);
        if constexpr (MODE == kGateKey) {
          store4(out + o, x[0], x[1], x[2], x[3]);
          store4(out + o + 4, x[4], x[5], x[6], x[7]);
        }
      }
    } else {
      constexpr int SPANS = G::BP / 4;             // 4-element spans per staged row
      for (int idx = threadIdx.x; idx < rows * SPANS; idx += G::NT) {
        const int r = idx / SPANS, c = (idx - r * SPANS) * 4;
        if (c >= pn) continue;                      // NP % 4 == 0
        const int64_t o = (int64_t)(q0 + ps * RPP + r) * g.ldo + p0 + c;
        f32x4 v = *reinterpret_cast<const f32x4*>(smem + st.off(r, c));
        if constexpr (MODE == kAccF32) v += load4(out + o);
        store4(out + o, v[0], v[1], v[2], v[3]);
        if constexpr (MODE == kStoreNeg)
          store4((T*)g.eo[0] + (int64_t)b * g.eo_so + o, -v[0], -v[1], -v[2], -v[3]);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- elementwise gate terms

struct EwArgs {
  const void *A, *U, *ddA, *ddU;   // [BH, C, m] each (contiguous)
  void* ddH;
  int64_t n;                       // elements per row group (C m)
};

// ddH = ddA U silu'(A) + ddU silu(A), eight consecutive elements per thread
// (the one gate stage that needs two GEMMs' outputs at once; the others are
// formed in the epilogue of the GEMM that produces their input).
template <typename T>
__global__ __launch_bounds__(256) void k_lact_ddh(EwArgs a) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e >= a.n) return;
  const int64_t o = (int64_t)blockIdx.y * a.n + e;
  auto ld8 = [&](const void* p, float* v) {
    const T* t = (const T*)p + o;
    const f32x4 x0 = load4(t), x1 = load4(t + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = x0[i];
      v[4 + i] = x1[i];
    }
  };
  float A[8], U[8], x1[8], x2[8], y[8];
  ld8(a.A, A);
  ld8(a.U, U);
  ld8(a.ddA, x1);
  ld8(a.ddU, x2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float s = sigmoid_f(A[i]);
    y[i] = x1[i] * U[i] * s * (1.0f + A[i] * (1.0f - s)) + x2[i] * A[i] * s;
  }
  T* t = (T*)a.ddH + o;
  store4(t, y[0], y[1], y[2], y[3]);
  store4(t + 4, y[4], y[5], y[6], y[7]);
}

// dst[bh][t][j] = 0 for one chunk's rows of a [BH, n, dh] buffer (dst already
// offset to the chunk; n elements per row group, row group stride dstride).
template <typename T>
__global__ __launch_bounds__(256) void k_lact_zero_rows(T* __restrict__ dst, int64_t n, int64_t dstride) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  store4(dst + (int64_t)blockIdx.y * dstride + e, 0.f, 0.f, 0.f, 0.f);
}


// gG = scale * g over the [BH, 3, m dh] gradients (operand dtype), four per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_lact_gscale(const float* __restrict__ g, T* __restrict__ out, int64_t n,
                                                     float scale) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  const f32x4 x = load4(g + e) * scale;
  store4(out + e, x[0], x[1], x[2], x[3]);
}

// g += sum over the nsplit partials part[s] (fp32, n elements each, splits in
// order), four elements per thread.
__global__ __launch_bounds__(256) void k_lact_gacc(const float* __restrict__ part, float* __restrict__ g, int64_t n,
                                                   int nsplit) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  f32x4 x = load4(g + e);
  for (int sp = 0; sp < nsplit; ++sp) x += load4(part + (int64_t)sp * n + e);
  store4(g + e, x[0], x[1], x[2], x[3]);
}

// out[h][e] = sum over the B rows of g[b H + h][w][e] (rows in order): the
// initial weights' gradients of head h; grid.y = h * 3 + w.
__global__ __launch_bounds__(256) void k_lact_gsum(const float* __restrict__ g, float* __restrict__ d1,
                                                   float* __restrict__ d3, float* __restrict__ d2, int B, int H,
                                                   int64_t md) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= md) return;
  const int h = blockIdx.y / 3, w = blockIdx.y % 3;
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) s += load4(g + (((int64_t)b * H + h) * 3 + w) * md + e);
  float* out = (w == 0 ? d1 : (w == 1 ? d3 : d2)) + (int64_t)h * md + e;
  store4(out, s[0], s[1], s[2], s[3]);
}

// ---------------------------------------------------------------- host side

// Workspace of the backward: the forward's own (for the recompute), the kept
// states, the fp32 state gradient and its scaled operand copy, the per-chunk
// intermediates and one fp32 [BH, C, dh] partial.
// The state gradient's contractions over a chunk's tokens are split at most
// this many ways (with 4 x 512 x 1024 states, three gradients of 32 tiles each
// would leave most of the GPU idle); the splits' fp32 partials are then added
// in order.
constexpr int kGradSplit = 4;

struct LactBwdWs {
  size_t fwd, keep, g, gG, cm[16], cd[2], gpart, total;
};

// saved: the forward call kept the states, so neither its workspace nor the
// state slots are needed here.
template <typename T>
LactBwdWs lact_bwd_layout(int B, int H, int n, int dh, int m, int C, bool saved = false) {
  LactBwdWs w{};
  const size_t e = sizeof(T), BH = (size_t)B * H, md = (size_t)m * dh, k = (size_t)(C > 0 ? n / C : 0);
  size_t o = 0;
  if (!saved) {
    w.fwd = o;
    o += al256(lact_workspace_bytes<T>(B, H, n, dh, m, C));
    w.keep = o;
    o += al256((k + 1) * BH * 3 * md * e);
  }
  w.g = o;
  o += al256(BH * 3 * md * 4);
  w.gG = o;
  o += al256(BH * 3 * md * e);
  for (int i = 0; i < 16; ++i) {
    w.cm[i] = o;
    o += al256(BH * (size_t)C * m * e);
  }
  for (int i = 0; i < 2; ++i) {
    w.cd[i] = o;
    o += al256(BH * (size_t)C * dh * e);
  }
  w.gpart = o;
  o += al256((size_t)kGradSplit * BH * 3 * md * 4);
  w.total = o;
  return w;
}

template <typename T, bool PMN, bool QMN, int NS, int MODE>
hipError_t bgemm_set(const BGemmSet& set, hipStream_t s) {
  int64_t tiles = 0;
  for (int i = 0; i < set.n; ++i)
    tiles += cdiv64(set.g[i].NP, Wide::BP) * cdiv64(set.g[i].NQ, Wide::BQ) * set.g[i].batch * set.nsplit;
  if (tiles == 0) return hipSuccess;
  k_bgemm<T, PMN, QMN, NS, MODE><<<(unsigned)tiles, Wide::NT, 0, s>>>(set);
  return hipGetLastError();
}

template <typename T, bool PMN, bool QMN, int NS, int MODE>
hipError_t bgemm(const BGemm& g, hipStream_t s) {
  if (g.NP <= 0 || g.NQ <= 0 || g.batch <= 0) return hipSuccess;
  BGemmSet set{};
  set.g[0] = g;
  set.n = 1;
  set.nsplit = 1;
  return bgemm_set<T, PMN, QMN, NS, MODE>(set, s);
}

// Two GEMMs of one kind as one launch (twice the tiles of either: the short-K
// products fill the GPU for two rounds instead of one).
template <typename T, bool PMN, bool QMN, int NS, int MODE>
hipError_t bgemm2(const BGemm& g0, const BGemm& g1, hipStream_t s) {
  BGemmSet set{};
  set.g[0] = g0;
  set.g[1] = g1;
  set.n = 2;
  set.nsplit = 1;
  return bgemm_set<T, PMN, QMN, NS, MODE>(set, s);
}

template <typename T>
hipError_t ddh(const EwArgs& a, int BH, hipStream_t s) {
  k_lact_ddh<T><<<dim3((unsigned)cdiv64(a.n / 8, 256), (unsigned)BH), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

template <typename T>
size_t lact_bwd_workspace_bytes(int B, int H, int n, int dh, int m, int C, bool saved) {
  return lact_bwd_layout<T>(B, H, n, dh, m, C, saved).total;
}

template <typename T>
hipError_t launch_lact_backward(const LactBwdArgs& a, hipStream_t s) {
  const int B = a.B, H = a.H, n = a.n, dh = a.dh, m = a.m, C = a.C;
  const int BH = B * H;
  const int64_t md = (int64_t)m * dh;
  hipError_t e;
  if (BH == 0) return hipSuccess;
  const bool saved = a.states != nullptr;
  const LactBwdWs L = lact_bwd_layout<T>(B, H, n, dh, m, C, saved);
  float* g = (float*)(a.ws + L.g);
  T* gG = (T*)(a.ws + L.gG);
  if ((e = launch_zero<float>(g, (int64_t)BH * 3 * md, s)) != hipSuccess) return e;
  if (n > 0 && !saved) {
    // the states: the forward's kernels on the keys alone, every chunk's state kept
    LactArgs f{};
    f.B = B;
    f.H = H;
    f.n = n;
    f.dh = dh;
    f.m = m;
    f.C = C;
    f.order = a.order;
    f.eta = a.eta;
    f.q = a.q;
    f.k = a.k;
    f.v = a.v;
    f.W1 = a.W1;
    f.W3 = a.W3;
    f.W2 = a.W2;
    f.O = nullptr;
    // the recompute's own final states land in the gradient buffer, cleared after it
    f.W1f = g;
    f.W3f = g + (int64_t)BH * md;
    f.W2f = g + 2 * (int64_t)BH * md;
    f.ws = a.ws + L.fwd;
    f.keys_only = 1;
    f.keep = a.ws + L.keep;
    f.update_mask = a.update_mask;
    if ((e = launch_lact<T>(f, s)) != hipSuccess) return e;
    if ((e = launch_zero<float>(g, (int64_t)BH * 3 * md, s)) != hipSuccess) return e;
  }
  const int k = C > 0 ? n / C : 0;
  const T* keep = saved ? (const T*)a.states : (const T*)(a.ws + L.keep);
  T* cm[16];
  for (int i = 0; i < 16; ++i) cm[i] = (T*)(a.ws + L.cm[i]);
  T* A = cm[0];
  T* U = cm[1];
  T* Hh = cm[2];
  T* dH = cm[3];
  T* dA = cm[4];
  T* dU = cm[5];
  T* ddA = cm[6];
  T* ddU = cm[7];
  T* ddH = cm[8];
  T* dAf = cm[9];
  T* dUf = cm[10];
  T* Aq = cm[11];
  T* Uq = cm[12];
  T* Hq = cm[13];
  T* dAq = cm[14];
  T* dUq = cm[15];
  T* R = (T*)(a.ws + L.cd[0]);
  T* dR = (T*)(a.ws + L.cd[1]);
  float* gpart = (float*)(a.ws + L.gpart);
  // the three state-gradient contractions of a phase, split over the tokens, then added into g
  // nsplit: 2 when the three have equal K (one round of 192 tiles at the workload), 4 when g2 has two K streams
  auto grad_set = [&](auto launch, int nsplit, BGemm g2, BGemm g1, BGemm g3) -> hipError_t {
    BGemmSet set{};
    set.g[0] = g2;
    set.g[1] = g1;
    set.g[2] = g3;
    set.n = 3;
    set.nsplit = nsplit;
    set.split_so = (int64_t)BH * 3 * md;
    hipError_t r = launch(set);
    if (r != hipSuccess) return r;
    const int64_t n = (int64_t)BH * 3 * md;
    k_lact_gacc<<<(unsigned)cdiv64(n / 4, 256), 256, 0, s>>>(gpart, g, n, nsplit);
    return hipGetLastError();
  };
  const int64_t S3 = 3 * md;                                 // row-group stride of states and gradients
  const int64_t Sn = (int64_t)n * dh, Scm = (int64_t)C * m, Scd = (int64_t)C * dh;
  // a [BH, C, x] intermediate as a K-major (token rows) or MN-major (tokens as K) operand
  auto cmK = [&](const T* p) { return BOp{p, m, Scm}; };
  auto cdK = [&](const T* p) { return BOp{p, dh, Scd}; };
  auto one = [&](BOp P, BOp Q, int K, int NP, int NQ, void* out, int64_t ldo, int64_t so, float alpha = 1.0f) {
    BGemm gm{};
    gm.P[0] = P;
    gm.Q[0] = Q;
    gm.K[0] = K;
    gm.NP = NP;
    gm.NQ = NQ;
    gm.batch = BH;
    gm.out = out;
    gm.ldo = ldo;
    gm.so = so;
    gm.alpha = alpha;
    return gm;
  };
  auto two = [&](BGemm gm, BOp P2, BOp Q2, int K2) {
    gm.P[1] = P2;
    gm.Q[1] = Q2;
    gm.K[1] = K2;
    return gm;
  };
  auto four = [&](BGemm gm, BOp P3, BOp Q3, int K3, BOp P4, BOp Q4, int K4) {
    gm.P[2] = P3;
    gm.Q[2] = Q3;
    gm.K[2] = K3;
    gm.P[3] = P4;
    gm.Q[3] = Q4;
    gm.K[3] = K4;
    return gm;
  };
  // dq of a chunk waits for the next dk launch, whose 128 tiles it fills up to one round (its dAq, dUq stay intact
  // until the next query pass, which launches a dq still pending on its own first)
  BGemm pending_dq{};
  bool dq_pending = false;
  auto flush_dq = [&]() -> hipError_t {
    if (!dq_pending) return hipSuccess;
    dq_pending = false;
    return bgemm<T, true, false, 4, kStoreT>(pending_dq, s);
  };

  // queries of a chunk applied with the state W (slot pointer, rows 3 m dh apart)
  auto query_backward = [&](const T* W, int c) -> hipError_t {
    const T *W1 = W, *W3 = W + md, *W2 = W + 2 * md;
    const BOp Qc{(const T*)a.q + (int64_t)c * C * dh, dh, Sn};
    const BOp dOc{(const T*)a.dO + (int64_t)c * C * dh, dh, Sn};
    hipError_t r;
    if ((r = flush_dq()) != hipSuccess) return r;
    // Aq, Uq and Hq by the forward's gate kernel; dHq = dO W2 with dAq, dUq formed in its epilogue
    if ((r = launch_lact_gate_pass<T>((const T*)a.q, W, S3, Aq, Uq, Hq, BH, n, dh, m, C, c, s)) != hipSuccess) return r;
    {
      BGemm gq = one({W2, m, S3}, dOc, dh, m, C, dAq, m, Scm);
      gq.in[0] = Aq;
      gq.in[1] = Uq;
      gq.eo[0] = dAq;
      gq.eo[1] = dUq;
      if ((r = bgemm<T, true, false, 1, kGateQ>(gq, s)) != hipSuccess) return r;
    }
    // g2 += dO^T Hq, g1 += dAq^T Q, g3 += dUq^T Q
    r = grad_set([&](const BGemmSet& set) { return bgemm_set<T, true, true, 1, kStoreF32>(set, s); }, 2,
                 one(cmK(Hq), dOc, C, m, dh, gpart + 2 * md, m, S3), one(Qc, cmK(dAq), C, dh, m, gpart, dh, S3),
                 one(Qc, cmK(dUq), C, dh, m, gpart + md, dh, S3));
    if (r != hipSuccess) return r;
    // dq = dAq W1 + dUq W3, launched with the next dk
    pending_dq = two(one({W1, dh, S3}, cmK(dAq), m, dh, C, (T*)a.dq + (int64_t)c * C * dh, dh, Sn), {W3, dh, S3},
                     cmK(dUq), m);
    dq_pending = true;
    return hipSuccess;
  };

  // the update of chunk c from the state W, upstream gG = -eta g
  auto update_backward = [&](const T* W, int c) -> hipError_t {
    const T *W1 = W, *W3 = W + md, *W2 = W + 2 * md;
    const T *gG1 = gG, *gG3 = gG + md, *gG2 = gG + 2 * md;
    const BOp Kc{(const T*)a.k + (int64_t)c * C * dh, dh, Sn};
    hipError_t r;
    k_lact_gscale<T><<<(unsigned)cdiv64((int64_t)BH * S3 / 4, 256), 256, 0, s>>>(g, gG, (int64_t)BH * S3, -a.eta);
    if ((r = hipGetLastError()) != hipSuccess) return r;
    // the forward's key pass at W: A, U, Hh by its gate kernel, R = Hh W2^T - v by its residual kernel (formed in
    // fp32, rounded once), then dH = R W2 with dA, dU formed in the epilogue
    if ((r = launch_lact_gate_pass<T>((const T*)a.k, W, S3, A, U, Hh, BH, n, dh, m, C, c, s)) != hipSuccess) return r;
    if ((r = launch_lact_residual_pass<T>(Hh, W, S3, (const T*)a.v, R, BH, n, dh, m, C, c, s)) != hipSuccess)
      return r;
    {
      BGemm gk = one({W2, m, S3}, cdK(R), dh, m, C, dH, m, Scm);
      gk.in[0] = A;
      gk.in[1] = U;
      gk.eo[0] = dA;
      gk.eo[1] = dU;
      if ((r = bgemm<T, true, false, 1, kGateKey>(gk, s)) != hipSuccess) return r;
    }
    // through G1 = dA^T k, G3 = dU^T k
    if ((r = bgemm2<T, false, false, 1, kStoreT>(one({gG1, dh, S3}, Kc, dh, m, C, ddA, m, Scm),
                                                 one({gG3, dh, S3}, Kc, dh, m, C, ddU, m, Scm), s)) != hipSuccess)
      return r;
    if ((r = ddh<T>(EwArgs{A, U, ddA, ddU, ddH, Scm}, BH, s)) != hipSuccess) return r;
    // dR = Hh gG2^T + ddH W2^T, and dv = -dR from the same epilogue
    {
      BGemm gr = two(one({gG2, m, S3}, cmK(Hh), m, dh, C, dR, dh, Scd), {W2, m, S3}, cmK(ddH), m);
      gr.eo[0] = (T*)a.dv + (int64_t)c * C * dh;
      gr.eo_so = Sn;
      if ((r = bgemm<T, false, false, 2, kStoreNeg>(gr, s)) != hipSuccess) return r;
    }
    // dHh = R gG2 + dR W2, never stored: dA_f and dU_f formed in the epilogue
    {
      BGemm gf = two(one({gG2, m, S3}, cdK(R), dh, m, C, dAf, m, Scm), {W2, m, S3}, cdK(dR), dh);
      gf.in[0] = A;
      gf.in[1] = U;
      gf.in[2] = dH;
      gf.in[3] = ddA;
      gf.in[4] = ddU;
      gf.eo[0] = dAf;
      gf.eo[1] = dUf;
      if ((r = bgemm<T, true, false, 2, kGateF>(gf, s)) != hipSuccess) return r;
    }
    // dk = dA gG1 + dU gG3 + dA_f W1 + dU_f W3: four K streams on one accumulator, rounded once into the
    // chunk's rows of dk (row group stride n dh); a pending dq (two streams) joins the launch
    {
      BGemmSet set{};
      set.g[0] = four(two(one({gG1, dh, S3}, cmK(dA), m, dh, C, (T*)a.dk + (int64_t)c * C * dh, dh, Sn), {gG3, dh, S3},
                          cmK(dU), m),
                      {W1, dh, S3}, cmK(dAf), m, {W3, dh, S3}, cmK(dUf), m);
      set.n = 1;
      set.nsplit = 1;
      if (dq_pending) {
        set.g[1] = pending_dq;
        set.n = 2;
        dq_pending = false;
      }
      if ((r = bgemm_set<T, true, false, 4, kStoreT>(set, s)) != hipSuccess) return r;
    }
    // g2 += R^T ddH + dR^T Hh, g1 += dA_f^T k, g3 += dU_f^T k (the last two as one-stream members of a
    // two-stream set: their second stream is empty)
    BGemm g1 = one(Kc, cmK(dAf), C, dh, m, gpart, dh, S3), g3 = one(Kc, cmK(dUf), C, dh, m, gpart + md, dh, S3);
    g1 = two(g1, g1.P[0], g1.Q[0], 0);
    g3 = two(g3, g3.P[0], g3.Q[0], 0);
    return grad_set([&](const BGemmSet& set) { return bgemm_set<T, true, true, 2, kStoreF32>(set, s); }, kGradSplit,
                    two(one(cmK(ddH), cdK(R), C, m, dh, gpart + 2 * md, m, S3), cmK(Hh), cdK(dR), C), g1, g3);
  };

  const int64_t slot = (int64_t)BH * S3;
  for (int c = k - 1; c >= 0; --c) {
    const T* Wc = keep + (int64_t)c * slot;
    const T* Wn = keep + (int64_t)(c + 1) * slot;
    if (a.order == 0 && (e = query_backward(Wn, c)) != hipSuccess) return e;
    if (a.update_mask == nullptr || a.update_mask[c] != 0) {
      if ((e = update_backward(Wc, c)) != hipSuccess) return e;
    } else {
      // no step: the state gradient passes through, and the chunk's keys and values reach nothing
      const dim3 gz((unsigned)cdiv64(Scd / 4, 256), (unsigned)BH);
      k_lact_zero_rows<T><<<gz, 256, 0, s>>>((T*)a.dk + (int64_t)c * C * dh, Scd, Sn);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      k_lact_zero_rows<T><<<gz, 256, 0, s>>>((T*)a.dv + (int64_t)c * C * dh, Scd, Sn);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.order != 0 && (e = query_backward(Wc, c)) != hipSuccess) return e;
  }
  if ((e = flush_dq()) != hipSuccess) return e;
  k_lact_gsum<<<dim3((unsigned)cdiv64(md / 4, 256), (unsigned)(3 * H)), 256, 0, s>>>(g, a.dW1, a.dW3, a.dW2, B, H, md);
  return hipGetLastError();
}

template size_t lact_bwd_workspace_bytes<float>(int, int, int, int, int, int, bool);
template size_t lact_bwd_workspace_bytes<bf16>(int, int, int, int, int, int, bool);
template hipError_t launch_lact_backward<float>(const LactBwdArgs&, hipStream_t);
template hipError_t launch_lact_backward<bf16>(const LactBwdArgs&, hipStream_t);

}  // namespace ttt
