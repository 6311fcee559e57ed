// LaCT SwiGLU fast-weight kernels for gfx950 (review of "Test-Time Training
// Done Right", LaCT Model Architecture §1, eq. (3)-(4); ordering of update and
// apply, same section).
//
// f_W(x) = W2 [silu(W1 x) * (W3 x)], per-chunk loss sum_i (1/2)||f_W(k_i) - v_i||^2,
// one plain GD step per chunk on (W1, W3, W2) together.  Every (batch row,
// head) pair -- "bh" below -- is an independent fast weight; each launch
// covers all of them.  For one chunk step, with X the rows [Q part; K part]
// that share the current weights (update-then-apply: queries of chunk c-1 and
// keys of chunk c; apply-then-update: queries and keys of chunk c):
//   fwd1   A = X W1^T, U = X W3^T, Hh = silu(A) * U        (keys: A and U kept)
//   fwd2   Y = Hh W2^T; queries: O = Y; keys: R = Y - V
//   dh     dH = R W2; dU = dH * silu(A); dA = dH * U * silu'(A)
//   grad   G1 = dA^T K, G3 = dU^T K, G2 = R^T Hh            (split over tokens)
//   update W -= eta * (sum of the splits), fp32 state plus operand copies
// Every intermediate is stored token-major ([tokens, features]); the weight
// gradients contract over tokens by reading them as MN-major operands
// (transposed in LDS), so no transposed copy is ever written.
// The bh rows are split into groups that run their chains of steps on
// separate streams (see launch_lact).
// Layouts: q, k, v, O [BH, n, dh]; W1, W3 [H, m, dh]; W2 [H, dh, m];
// states W1f, W3f [BH, m, dh], W2f [BH, dh, m] (fp32).
#include <type_traits>

#include "gemm.hpp"
#include "launch.hpp"

namespace ttt {

namespace {

template <typename T> constexpr int esz() { return (int)sizeof(T); }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr int kSplit = 2;              // token splits of the weight-gradient GEMMs

// Workspace layout (byte offsets), one region per buffer.
struct LactWs {
  size_t Hh, A, U, R, dA, dU, W1s, W3s, W2s, part, mX0, mX1, mA, mB, mnorm, total;
};

constexpr int kMuonNormBlocks = 64;     // partial sums of squares per gradient

inline size_t al(size_t x) { return (x + 255) / 256 * 256; }

template <typename T>
LactWs lact_layout(int bh_rows, int dh, int m, int C) {
  const size_t e = sizeof(T), BH = (size_t)bh_rows, md = (size_t)m * dh;
  LactWs w{};
  size_t o = 0;
  w.Hh = o;   o += al(2 * BH * C * m * e);        // hidden of [Q part; K part] [2, BH, C, m]
  w.A = o;    o += al(BH * C * m * e);            // key pre-activations [BH, C, m]
  w.U = o;    o += al(BH * C * m * e);
  w.R = o;    o += al(BH * C * dh * e);           // residual f(k) - v [BH, C, dh]
  w.dA = o;   o += al(BH * C * m * e);            // gate backward [BH, C, m]
  w.dU = o;   o += al(BH * C * m * e);
  w.W1s = o;  o += al(BH * md * e);               // operand copies of the current state
  w.W3s = o;  o += al(BH * md * e);
  w.W2s = o;  o += al(BH * md * e);
  w.part = o; o += al((size_t)kSplit * BH * 3 * md * 4);   // split-token gradient partials
  // Muon: iterates X (two, ping-pong) [3 BH, r, c], A and B [3 BH, r, r], norm partials
  const size_t r = (size_t)(m < dh ? m : dh);
  w.mX0 = o;  o += al(3 * BH * md * e);
  w.mX1 = o;  o += al(3 * BH * md * e);
  w.mA = o;   o += al(3 * BH * r * r * e);
  w.mB = o;   o += al(3 * BH * r * r * e);
  w.mnorm = o; o += al(3 * BH * kMuonNormBlocks * 4);
  w.total = o;
  return w;
}

}  // namespace

// Rows of a chunk step: part 0 = queries of chunk qc (nq rows), part 1 = keys of
// chunk kc (nk rows).  Row tiles never straddle the parts.
struct StepRows {
  int nq, nk, qc, kc;
};

__host__ __device__ constexpr int cdiv_d(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------ fwd1

// A = X W1^T, U = X W3^T over the rows X of both parts.  P = W1 / W3 rows in
// alternating 32-row blocks (128 hidden units per tile), Q = rows (tokens),
// so that a lane holds 4 consecutive hidden units of one token.  Writes Hh
// [2, BH, C, m] for both parts (part p of row bh at Hh + p hpart + bh C m),
// and for the key part A and U [BH, C, m].  Row bh's W1 and W3 are at W1s +
// bh wsb and W3s + bh wsb.
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_lact_fwd1(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ W1s,
                                       const T* __restrict__ W3s, T* __restrict__ Hh, T* __restrict__ A,
                                       T* __restrict__ U, int BH, int n, int dh, int m, int C, StepRows sr,
                                       int64_t wsb, int64_t hpart) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (m + G::BP / 2 - 1) / (G::BP / 2);
  const int tqq = (sr.nq + G::BQ - 1) / G::BQ, tqk = (sr.nk + G::BQ - 1) / G::BQ;
  const int TQ = tqq + tqk, per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / per;
  int tp, tq;
  grouped_tile(id - bh * per, TP, TQ, 4, tp, tq);
  const int part = tq < tqq ? 0 : 1;
  const int r0 = (part ? tq - tqq : tq) * G::BQ;
  const int nrows = part ? sr.nk : sr.nq;
  const T* X = (part ? k : q) + ((int64_t)bh * n + (int64_t)(part ? sr.kc : sr.qc) * C) * dh;
  const int j0 = tp * (G::BP / 2);
  const uint64_t ldb = (uint64_t)dh * esz<T>();
  const int64_t md = (int64_t)m * dh;

  DmaOp<G::NW, G::BP, true> op;
  op.init(W1s + bh * wsb + (int64_t)j0 * dh, W3s + bh * wsb + (int64_t)j0 * dh, min(G::BP / 2, m - j0), ldb,
          (unsigned)ldb);
  DmaOp<G::NW, G::BQ> oq;
  oq.init(X + (int64_t)r0 * dh, nullptr, min(G::BQ, nrows - r0), ldb, (unsigned)ldb);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  // Tile row r holds W1 row ((r >> 6) << 5) + (r & 31) in even 32-row blocks and
  // the same W3 row in odd ones, so a wave's P blocks 0, 1, 4, 5 are W1 rows and
  // block i + 2 holds the W3 rows of block i.  Every output is a [token][hidden]
  // tile staged in LDS and copied out as whole row pieces: A and U of the keys
  // together (one half of the stage area each, when they fit), then
  // Hh = silu(A) * U, formed in place of A.
  static_assert(G::NPB == 8 && G::BM == 16 && G::GPB == 1 && G::BP / G::WP == 128,
                "two W1/W3 block pairs per 32 rows of a wave");
  using ST = Staged<T, G::BP / 2>;
  constexpr int TILE = G::BQ * ST::RB;                           // bytes of one staged output
  constexpr bool PAIR = 2 * TILE <= G::Smem;
  const int jn = min(G::BP / 2, m - j0), tn = min(G::BQ, nrows - r0);
  auto hcol = [](int i) {                                        // local hidden unit of W1 block i
    const int r = G::acc_p(i, 0);
    return ((r >> 6) << 5) + (r & 31);
  };
  // half: 0 = W1 blocks (A, later Hh), 2 = W3 blocks (U); a compile-time
  // constant, so that the accumulators stay in registers
  auto put = [&](char* base, auto half) __attribute__((always_inline)) {
    const ST st{base};
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = (ii & 1) + 4 * (ii >> 1);                    // 0, 1, 4, 5
#pragma unroll
      for (int j = 0; j < G::NQB; ++j) {
        const f32x4& v = acc[i + decltype(half)::value][j];
        st.put4(G::acc_q(j), hcol(i), v[0], v[1], v[2], v[3]);
      }
    }
  };
  auto flush = [&](char* base, T* dst) __attribute__((always_inline)) {   // dst: [C, m] block of this bh
    const ST st{base};
    st.template flush<G::NT, G::BQ>(tn, [&](int r, int col) -> T* {
      return col < jn ? dst + (int64_t)(r0 + r) * m + j0 + col : nullptr;
    });
  };
  using H0 = std::integral_constant<int, 0>;
  using H2 = std::integral_constant<int, 2>;
  if (part) {
    T* a_ = A + (int64_t)bh * C * m;
    T* u_ = U + (int64_t)bh * C * m;
    if constexpr (PAIR) {
      put(smem, H0{});
      put(smem + TILE, H2{});
      __syncthreads();
      flush(smem, a_);
      flush(smem + TILE, u_);
      __syncthreads();
    } else {
      put(smem, H0{});
      __syncthreads();
      flush(smem, a_);
      __syncthreads();
      put(smem, H2{});
      __syncthreads();
      flush(smem, u_);
      __syncthreads();
    }
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int i = (ii & 1) + 4 * (ii >> 1);
#pragma unroll
    for (int j = 0; j < G::NQB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = silu_f(acc[i][j][e]) * acc[i + 2][j][e];
  }
  put(smem, H0{});
  __syncthreads();
  flush(smem, Hh + (int64_t)part * hpart + (int64_t)bh * C * m);
}

// ------------------------------------------------------------------ fwd2

// Y = Hh W2^T.  P = dh rows of W2s (row bh's [dh, m] at W2s + bh wsb), Q =
// rows of Hh (both parts, laid out as k_lact_fwd1 writes them).
// Query rows: O[bh, qc C + r, :] = Y.  Key rows: R [BH, C, dh], the gradient of
// the chunk loss with respect to the output -- Y - V for the squared error,
// -V for the dot-product loss (loss_dot) -- times the token's learning rate
// eta_tok [BH, n] when given (LaCT Model Architecture §1, eq. (3)).
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_lact_fwd2(const T* __restrict__ Hh, const T* __restrict__ W2s, const T* __restrict__ v,
                                       T* __restrict__ O, T* __restrict__ R, int BH, int n, int dh, int m, int C,
                                       StepRows sr, const float* __restrict__ eta_tok, int loss_dot, int64_t wsb,
                                       int64_t hpart) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (dh + G::BP - 1) / G::BP;
  const int tqq = (sr.nq + G::BQ - 1) / G::BQ, tqk = (sr.nk + G::BQ - 1) / G::BQ;
  const int TQ = tqq + tqk, per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / per;
  int tp, tq;
  grouped_tile(id - bh * per, TP, TQ, 4, tp, tq);
  const int part = tq < tqq ? 0 : 1;
  const int r0 = (part ? tq - tqq : tq) * G::BQ;
  const int nrows = part ? sr.nk : sr.nq;
  const int i0 = tp * G::BP;
  const uint64_t ldb = (uint64_t)m * esz<T>();

  DmaOp<G::NW, G::BP> op;
  DmaOp<G::NW, G::BQ> oq;
  op.init(W2s + (int64_t)bh * wsb + (int64_t)i0 * m, nullptr, min(G::BP, dh - i0), ldb, (unsigned)ldb);
  oq.init(Hh + (int64_t)part * hpart + ((int64_t)bh * C + r0) * m, nullptr, min(G::BQ, nrows - r0), ldb,
          (unsigned)ldb);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  static_assert(G::GPB == 1, "one accumulator group per block");
  const int tn = min(G::BQ, nrows - r0), in_ = min(G::BP, dh - i0);
  constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(T) + G::Smem - 1) / G::Smem, RPP = G::BQ / PASSES;
  // O (queries) or R = Y - V (keys, formed in fp32 block by block), [token][channel]:
  // staged by token rows.
  const Staged<T, G::BP> st{smem};
  T* base = part ? R + (int64_t)bh * C * dh : O + ((int64_t)bh * n + (int64_t)sr.qc * C) * dh;
  if (part) {
    // R in the accumulators before any staging, so that the loads of V and of
    // the rates are not held up behind LDS traffic; a lane outside the matrix
    // reads the nearest valid element of V (never stored)
#pragma unroll
    for (int jq = 0; jq < G::NQB; ++jq) {
      const int r = min(r0 + G::acc_q(jq), nrows - 1);
      const int64_t tok = (int64_t)bh * n + (int64_t)sr.kc * C + r;
      const float rate = eta_tok != nullptr ? eta_tok[tok] : 1.0f;
#pragma unroll
      for (int ib = 0; ib < G::NPB; ++ib) {
        const int i = min(i0 + G::acc_p(ib, 0), dh - 4);
        const f32x4 vv = load4(v + tok * dh + i);
        f32x4& y = acc[ib][jq];
        y = loss_dot ? -vv : y - vv;
        y *= rate;
      }
    }
  }
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int jq = 0; jq < G::NQB; ++jq) {
      const int q = G::acc_q(jq) - ps * RPP;
      if (q < 0 || q >= RPP) continue;
#pragma unroll
      for (int ib = 0; ib < G::NPB; ++ib)
        st.put4(q, G::acc_p(ib, 0), acc[ib][jq][0], acc[ib][jq][1], acc[ib][jq][2], acc[ib][jq][3]);
    }
    __syncthreads();
    const int rows = max(0, min(RPP, tn - ps * RPP));
    st.template flush<G::NT, RPP>(rows, [&](int rr, int col) -> T* {
      return col < in_ ? base + (int64_t)(r0 + ps * RPP + rr) * dh + i0 + col : nullptr;
    });
    __syncthreads();
  }
}

// ------------------------------------------------------------------ dh

// dH = R W2 [C, m]; P = m (W2s [BH, dh, m] read as an MN-major operand), Q =
// tokens (R rows).  Epilogue, the SiLU-gate backward: dH is staged as fp32
// [token][m] rows (in passes over tokens); each thread then takes 8
// consecutive m of one token, reads A and U in 16-byte pieces and writes
// dU = dH * silu(A), dA = dH * U * silu'(A), silu'(a) = s (1 + a (1 - s)),
// s = sigmoid(a), the same way ([BH, C, m]).
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_lact_dh(const T* __restrict__ R, const T* __restrict__ W2s, const T* __restrict__ A,
                                     const T* __restrict__ U, T* __restrict__ dA, T* __restrict__ dU, int BH, int dh,
                                     int m, int C, int nk) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (m + G::BP - 1) / G::BP, TQ = (nk + G::BQ - 1) / G::BQ, per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / per;
  int tp, tq;
  grouped_tile(id - bh * per, TP, TQ, 4, tp, tq);
  const int j0 = tp * G::BP, t0 = tq * G::BQ;
  const uint64_t ldb = (uint64_t)dh * esz<T>();

  DmaOpMN<T, G::NW, G::BP> op;
  DmaOp<G::NW, G::BQ> oq;
  op.init(W2s + (int64_t)bh * dh * m + j0, min(G::BP, m - j0), (uint64_t)m * esz<T>(), dh);
  oq.init(R + ((int64_t)bh * C + t0) * dh, nullptr, min(G::BQ, nk - t0), ldb, (unsigned)ldb);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  static_assert(G::GPB == 1, "one accumulator group per block");
  const int jn = min(G::BP, m - j0), tn = min(G::BQ, nk - t0);
  constexpr int RPP = G::Smem / (G::BP * 4);        // token rows per pass
  constexpr int PASSES = G::BQ / RPP;
  constexpr int SPANS = G::BP / 8;                  // 8-column spans per row
  const Staged<float, G::BP> st{smem};
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int jq = 0; jq < G::NQB; ++jq) {
      const int qq = G::acc_q(jq) - ps * RPP;
      if (qq < 0 || qq >= RPP) continue;
#pragma unroll
      for (int ib = 0; ib < G::NPB; ++ib)
        st.put4(qq, G::acc_p(ib, 0), acc[ib][jq][0], acc[ib][jq][1], acc[ib][jq][2], acc[ib][jq][3]);
    }
    __syncthreads();
    const int rows = max(0, min(RPP, tn - ps * RPP));
    for (int idx = threadIdx.x; idx < rows * SPANS; idx += G::NT) {
      const int r = idx / SPANS, c = (idx - r * SPANS) * 8;
      if (c >= jn) continue;                            // jn % 8 == 0
      const int64_t o = ((int64_t)bh * C + t0 + ps * RPP + r) * m + j0 + c;
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(smem + st.off(r, c));
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(smem + st.off(r, c + 4));
      const f32x4 a0 = load4(A + o), a1 = load4(A + o + 4), u0 = load4(U + o), u1 = load4(U + o + 4);
      float du[8], da[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = e < 4 ? d0[e] : d1[e - 4];
        const float a = e < 4 ? a0[e] : a1[e - 4];
        const float u = e < 4 ? u0[e] : u1[e - 4];
        const float s = sigmoid_f(a);
        du[e] = g * a * s;
        da[e] = g * u * s * (1.0f + a * (1.0f - s));
      }
      store4(dU + o, du[0], du[1], du[2], du[3]);
      store4(dU + o + 4, du[4], du[5], du[6], du[7]);
      store4(dA + o, da[0], da[1], da[2], da[3]);
      store4(dA + o + 4, da[4], da[5], da[6], da[7]);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ weight gradients

// Three contractions over the chunk's tokens, split kSplit ways along the
// tokens, written as fp32 partials part[s][bh][w] (w = 0: G1 [m, dh], 1: G3
// [m, dh], 2: G2 [dh, m]).  Every operand is token-major and read as an
// MN-major operand (k = tokens):
//   G1[j][i] = sum_t dA[t][j] K[t][i]   P = i (K columns), Q = j (dA columns)
//   G3[j][i] = sum_t dU[t][j] K[t][i]   P = i (K columns), Q = j (dU columns)
//   G2[i][j] = sum_t R[t][i] Hh[t][j]   P = j (Hh columns), Q = i (R columns)
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_lact_grad(const T* __restrict__ k, const T* __restrict__ dA, const T* __restrict__ dU,
                                       const T* __restrict__ Hh, const T* __restrict__ R, float* __restrict__ part,
                                       int BH, int n, int dh, int m, int C, int kc, int nk, int kslice) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int tA = cdiv_d(dh, G::BP) * cdiv_d(m, G::BQ);   // tiles of G1 and of G3
  const int tB = cdiv_d(m, G::BP) * cdiv_d(dh, G::BQ);   // tiles of G2
  const int per = 2 * tA + tB;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int sb = id / per;
  int r = id - sb * per;
  const int s = sb % kSplit, bh = sb / kSplit;
  const int which = r < tA ? 0 : (r < 2 * tA ? 1 : 2);
  r -= which == 0 ? 0 : (which == 1 ? tA : 2 * tA);
  const int PD = which < 2 ? dh : m, QD = which < 2 ? m : dh;     // P and Q extents
  int tp, tq;
  grouped_tile(r, cdiv_d(PD, G::BP), cdiv_d(QD, G::BQ), 4, tp, tq);
  const int p0 = tp * G::BP, q0 = tq * G::BQ;
  const int tk0 = s * kslice;
  const int kl = max(0, min(kslice, nk - tk0));
  const T* Pbase;
  const T* Qbase;
  if (which < 2) {
    Pbase = k + ((int64_t)bh * n + (int64_t)kc * C + tk0) * dh + p0;
    Qbase = (which == 0 ? dA : dU) + ((int64_t)bh * C + tk0) * m + q0;
  } else {
    Pbase = Hh + ((int64_t)(BH + bh) * C + tk0) * m + p0;         // key part of Hh
    Qbase = R + ((int64_t)bh * C + tk0) * dh + q0;
  }
  DmaOpMN<T, G::NW, G::BP> op;
  DmaOpMN<T, G::NW, G::BQ> oq;
  op.init(Pbase, min(G::BP, PD - p0), (uint64_t)PD * esz<T>(), kl);
  oq.init(Qbase, min(G::BQ, QD - q0), (uint64_t)QD * esz<T>(), kl);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  constexpr int KR = 128 / esz<T>();
  mainloop<T, G>(op, oq, (kl + KR - 1) / KR, acc, smem, NoHook{});
  const int64_t md = (int64_t)m * dh;
  float* out = part + (((int64_t)s * BH + bh) * 3 + which) * md;
#pragma unroll
  for (int jq = 0; jq < G::NQB; ++jq) {
    const int qi = q0 + G::acc_q(jq);
    if (qi >= QD) continue;
#pragma unroll
    for (int ib = 0; ib < G::NPB; ++ib)
#pragma unroll
      for (int g = 0; g < G::GPB; ++g) {
        const int pi = p0 + G::acc_p(ib, g);
        if (pi < PD)
          store4(out + (int64_t)qi * PD + pi, acc[ib][jq][4 * g], acc[ib][jq][4 * g + 1], acc[ib][jq][4 * g + 2],
                 acc[ib][jq][4 * g + 3]);
      }
  }
}

// ------------------------------------------------------------------ state update

// W -= eta * sum_s part[s]; writes the fp32 state and the operand copies.
// Four elements per thread; grid.y = bh * 3 + w.
template <typename T>
__global__ __launch_bounds__(256) void k_lact_update(const float* __restrict__ part, float* __restrict__ W1f,
                                                     float* __restrict__ W3f, float* __restrict__ W2f,
                                                     T* __restrict__ W1s, T* __restrict__ W3s, T* __restrict__ W2s,
                                                     int BH, int dh, int m, float eta) {
  const int64_t md = (int64_t)m * dh;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= md) return;
  const int bh = blockIdx.y / 3, w = blockIdx.y % 3;
  f32x4 gsum = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kSplit; ++s) gsum += load4(part + (((int64_t)s * BH + bh) * 3 + w) * md + e);
  float* Wf = (w == 0 ? W1f : (w == 1 ? W3f : W2f)) + (int64_t)bh * md + e;
  T* Ws = (w == 0 ? W1s : (w == 1 ? W3s : W2s)) + (int64_t)bh * md + e;
  f32x4 x = load4(Wf);
  x -= eta * gsum;
  store4(Wf, x[0], x[1], x[2], x[3]);
  store4(Ws, x[0], x[1], x[2], x[3]);
}

// L2 weight normalisation after an update (LaCT Model Architecture §2): every
// row of W1, W3 [m, dh] and of W2 [dh, m] -- each matrix's input dimension -- is
// scaled to unit norm, in the fp32 state and its operand copy.  One wave per
// row; grid.x covers 4 rows per block, grid.y = 3 BH (matrix w of row bh).
template <typename T>
__global__ __launch_bounds__(256) void k_lact_wnorm(float* __restrict__ W1f, float* __restrict__ W3f,
                                                    float* __restrict__ W2f, T* __restrict__ W1s, T* __restrict__ W3s,
                                                    T* __restrict__ W2s, int dh, int m) {
  const int bh = blockIdx.y / 3, w = blockIdx.y % 3;
  const int rows = w == 2 ? dh : m, len = w == 2 ? m : dh;
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t o = (int64_t)bh * m * dh + (int64_t)row * len;
  float* Wf = (w == 0 ? W1f : (w == 1 ? W3f : W2f)) + o;
  T* Ws = (w == 0 ? W1s : (w == 1 ? W3s : W2s)) + o;
  float ss = 0.f;
  for (int i = lane * 4; i < len; i += 256) {
    const f32x4 x = load4(Wf + i);
    ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
  for (int i = lane * 4; i < len; i += 256) {
    const f32x4 x = load4(Wf + i) * inv;
    store4(Wf + i, x[0], x[1], x[2], x[3]);
    store4(Ws + i, x[0], x[1], x[2], x[3]);
  }
}

// ------------------------------------------------------------------ Muon

// The Muon update rule (LaCT Model Architecture §2): each gradient g is replaced
// by Muon(g) ~ U V^T before the step.  The page names Newton-Schulz without its
// polynomial; this is the quintic iteration with the coefficients published
// with the Muon optimizer: X = g / ||g||_F in the wide orientation [r, c]
// (r = min(m, dh), c = max(m, dh)), then five times A = X X^T,
// B = b A + c A^2, X <- a X + B X, stored in the operand dtype with fp32
// accumulation.  The 3 BH gradients of a step (matrix mat = 3 bh + w) form one
// batch.
constexpr float kMuonA = 3.4445f, kMuonB = -4.7750f, kMuonC = 2.0315f;
constexpr int kMuonSteps = 5;

// Gradient w is [m, dh] for W1, W3 and [dh, m] for W2; tall ones are iterated
// transposed.
__host__ __device__ inline bool muon_tall(int w, int dh, int m) { return w < 2 ? m > dh : dh > m; }

// Partial sums of squares of g (the sum of the split partials), kMuonNormBlocks
// per gradient.
__global__ __launch_bounds__(256) void k_muon_norm(const float* __restrict__ part, float* __restrict__ normp, int BH,
                                                   int64_t md) {
  const int mat = blockIdx.y, bh = mat / 3, w = mat % 3;
  float ss = 0.f;
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < md; e += (int64_t)kMuonNormBlocks * 1024) {
    f32x4 g = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSplit; ++s) g += load4(part + (((int64_t)s * BH + bh) * 3 + w) * md + e);
    ss += g[0] * g[0] + g[1] * g[1] + g[2] * g[2] + g[3] * g[3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  __shared__ float wsum[4];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) normp[mat * kMuonNormBlocks + blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// X0 = g / (||g||_F + 1e-7) in the wide orientation [r, c], one element per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_muon_prep(const float* __restrict__ part, const float* __restrict__ normp,
                                                   T* __restrict__ X, int BH, int dh, int m) {
  const int mat = blockIdx.y, bh = mat / 3, w = mat % 3;
  const int r = m < dh ? m : dh, c = m < dh ? dh : m;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x, md = (int64_t)m * dh;
  if (idx >= md) return;
  const int i = (int)(idx / c), j = (int)(idx % c);
  float ss = 0.f;
  for (int t = 0; t < kMuonNormBlocks; ++t) ss += normp[mat * kMuonNormBlocks + t];
  const float inv = 1.0f / (sqrtf(ss) + 1e-7f);
  // g is [c, r] when tall (X = g^T), else [r, c]
  const int64_t ge = muon_tall(w, dh, m) ? (int64_t)j * r + i : (int64_t)i * c + j;
  float g = 0.f;
#pragma unroll
  for (int s = 0; s < kSplit; ++s) g += part[(((int64_t)s * BH + bh) * 3 + w) * md + ge];
  X[(int64_t)mat * md + idx] = from_f32<T>(g * inv);
}

// One GEMM of a Newton-Schulz step for every gradient of the batch (grid.y):
//   STEP 0: A = X X^T                  P = X rows,            Q = X rows,  K = c
//   STEP 1: B = b A + c A A^T (= A^2)  P = A rows,            Q = A rows,  K = r
//   STEP 2: Xn = a X + B X             P = X columns (MN),    Q = B rows,  K = r
// Output row-major, rows indexed by Q and columns by P, so that a lane's four
// accumulators are four consecutive elements of one row.
// The matrices are small (a few hundred 256 x 256 tiles at most over all of a
// step's gradients), so the GEMMs take the 128 x 128 tile of 4 waves, two
// workgroups per CU (register budget of two waves per SIMD).
template <typename T, int STEP>
__global__ __launch_bounds__(Half::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ns_gemm(
    const T* __restrict__ X, const T* __restrict__ A, const T* __restrict__ Bm, T* __restrict__ out, int r, int c) {
  using G = Half;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int mat = blockIdx.y;
  const int cols = STEP == 2 ? c : r, rows = r;
  const int TP = (cols + G::BP - 1) / G::BP, TQ = (rows + G::BQ - 1) / G::BQ;
  int tp, tq;
  grouped_tile((int)blockIdx.x, TP, TQ, 4, tp, tq);
  const int p0 = tp * G::BP, q0 = tq * G::BQ;
  const T* x = X + (int64_t)mat * r * c;
  const T* a = A + (int64_t)mat * r * r;
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  if constexpr (STEP == 0) {
    const uint64_t ld = (uint64_t)c * esz<T>();
    DmaOp<G::NW, G::BP> op;
    DmaOp<G::NW, G::BQ> oq;
    op.init(x + (int64_t)p0 * c, nullptr, min(G::BP, cols - p0), ld, (unsigned)ld);
    oq.init(x + (int64_t)q0 * c, nullptr, min(G::BQ, rows - q0), ld, (unsigned)ld);
    mainloop<T, G>(op, oq, (int)((ld + 127) / 128), acc, smem, NoHook{});
  } else if constexpr (STEP == 1) {
    const uint64_t ld = (uint64_t)r * esz<T>();
    DmaOp<G::NW, G::BP> op;
    DmaOp<G::NW, G::BQ> oq;
    op.init(a + (int64_t)p0 * r, nullptr, min(G::BP, cols - p0), ld, (unsigned)ld);
    oq.init(a + (int64_t)q0 * r, nullptr, min(G::BQ, rows - q0), ld, (unsigned)ld);
    mainloop<T, G>(op, oq, (int)((ld + 127) / 128), acc, smem, NoHook{});
  } else {
    const uint64_t ld = (uint64_t)r * esz<T>();
    DmaOpMN<T, G::NW, G::BP> op;
    DmaOp<G::NW, G::BQ> oq;
    op.init(x + p0, min(G::BP, cols - p0), (uint64_t)c * esz<T>(), r);
    oq.init(Bm + (int64_t)mat * r * r + (int64_t)q0 * r, nullptr, min(G::BQ, rows - q0), ld, (unsigned)ld);
    mainloop<T, G>(op, oq, (r + DmaOpMN<T, G::NW, G::BP>::KR - 1) / DmaOpMN<T, G::NW, G::BP>::KR, acc, smem,
                   NoHook{});
  }
  T* o = out + (int64_t)mat * rows * cols;
#pragma unroll
  for (int jq = 0; jq < G::NQB; ++jq) {
    const int q = q0 + G::acc_q(jq);
    if (q >= rows) continue;
#pragma unroll
    for (int ib = 0; ib < G::NPB; ++ib) {
      const int p = p0 + G::acc_p(ib, 0);
      if (p >= cols) continue;                          // cols % 8 == 0: p .. p + 3 inside
      f32x4 v = acc[ib][jq];
      if constexpr (STEP == 1) v = kMuonC * v + kMuonB * load4(a + (int64_t)q * r + p);
      if constexpr (STEP == 2) v = v + kMuonA * load4(x + (int64_t)q * c + p);
      store4(o + (int64_t)q * cols + p, v[0], v[1], v[2], v[3]);
    }
  }
}

// W -= eta Muon(g): the final iterate X, transposed back for tall gradients;
// fp32 state and its operand copy, four elements per thread, grid.y = 3 BH.
template <typename T>
__global__ __launch_bounds__(256) void k_lact_update_muon(const T* __restrict__ X, float* __restrict__ W1f,
                                                          float* __restrict__ W3f, float* __restrict__ W2f,
                                                          T* __restrict__ W1s, T* __restrict__ W3s,
                                                          T* __restrict__ W2s, int dh, int m, float eta) {
  const int64_t md = (int64_t)m * dh;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= md) return;
  const int mat = blockIdx.y, bh = mat / 3, w = mat % 3;
  const int cw_ = w == 2 ? m : dh;                     // columns of W (and of g)
  const int c = m < dh ? dh : m;
  const T* x = X + (int64_t)mat * md;
  f32x4 u;
  if (muon_tall(w, dh, m)) {                          // W[i][j] -= eta X[j][i]
    const int i = (int)(e / cw_), j = (int)(e % cw_);
#pragma unroll
    for (int t = 0; t < 4; ++t) u[t] = to_f32(x[(int64_t)(j + t) * c + i]);
  } else {
    u = load4(x + e);
  }
  float* Wf = (w == 0 ? W1f : (w == 1 ? W3f : W2f)) + (int64_t)bh * md + e;
  T* Ws = (w == 0 ? W1s : (w == 1 ? W3s : W2s)) + (int64_t)bh * md + e;
  f32x4 v = load4(Wf);
  v -= eta * u;
  store4(Wf, v[0], v[1], v[2], v[3]);
  store4(Ws, v[0], v[1], v[2], v[3]);
}

// Initial state of every (batch row, head) of a group that starts at row bh0,
// from the heads' initial weights.
template <typename T>
__global__ __launch_bounds__(256) void k_lact_init(const T* __restrict__ W1, const T* __restrict__ W3,
                                                   const T* __restrict__ W2, float* __restrict__ W1f,
                                                   float* __restrict__ W3f, float* __restrict__ W2f,
                                                   T* __restrict__ W1s, T* __restrict__ W3s, T* __restrict__ W2s,
                                                   int bh0, int H, int dh, int m) {
  const int64_t md = (int64_t)m * dh;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= md) return;
  const int bh = blockIdx.y / 3, w = blockIdx.y % 3, h = (bh0 + bh) % H;
  const T* src = (w == 0 ? W1 : (w == 1 ? W3 : W2)) + (int64_t)h * md + e;
  const f32x4 x = load4(src);
  float* Wf = (w == 0 ? W1f : (w == 1 ? W3f : W2f)) + (int64_t)bh * md + e;
  T* Ws = (w == 0 ? W1s : (w == 1 ? W3s : W2s)) + (int64_t)bh * md + e;
  store4(Wf, x[0], x[1], x[2], x[3]);
  store4(Ws, x[0], x[1], x[2], x[3]);
}

// A row group's operand copies (W1, W3, W2) into a kept-state slot [BH, 3, m dh],
// four elements per thread; grid.y = bh * 3 + w.
template <typename T>
__global__ __launch_bounds__(256) void k_lact_keep(const T* __restrict__ W1s, const T* __restrict__ W3s,
                                                   const T* __restrict__ W2s, T* __restrict__ dst, int64_t md) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= md) return;
  const int bh = blockIdx.y / 3, w = blockIdx.y % 3;
  const T* src = (w == 0 ? W1s : (w == 1 ? W3s : W2s)) + (int64_t)bh * md + e;
  const f32x4 x = load4(src);
  store4(dst + (int64_t)blockIdx.y * md + e, x[0], x[1], x[2], x[3]);
}

// ------------------------------------------------------------------ host driver

// The chunk steps of one (batch, head) row are a chain of short launches, each
// MFMA-bound in its K loop and HBM-bound in its epilogue, and one workgroup
// fills a CU.  The rows are therefore split into kGroups groups whose chains
// run on separate streams: the hardware then runs one group's epilogues and
// small launches beside another group's K loops.  Each group has its own
// region of the workspace.  Group 0 enqueues its first kLead launches (the
// init and the forward launches of its first step) before the others start,
// so that the groups run about half a step apart instead of in lockstep.
// (256K tokens, 4 heads: 17.1 ms with one group, 16.7 with two, 16.5 with two
// and the lead; four groups of one head each are much slower.)
constexpr int kGroups = 2;
constexpr int kLead = 3;

inline int group_rows(int BH, int G, int g) { return BH / G + (g < BH % G ? 1 : 0); }

template <typename T>
size_t lact_workspace_bytes(int B, int H, int n, int dh, int m, int C) {
  (void)n;
  const int BH = B * H, G = BH < kGroups ? (BH > 0 ? BH : 1) : kGroups;
  size_t total = 0;
  for (int g = 0; g < G; ++g) total += lact_layout<T>(group_rows(BH, G, g), dh, m, C).total;
  return total;
}

namespace {

// One group: rows [bh0, bh0 + BH) of the call, with its workspace region;
// only its launches first .. last - 1 (in enqueue order) are enqueued.
template <typename T>
hipError_t enqueue_lact_group(const LactArgs& a, int bh0, int BH, char* wsg, hipStream_t s, int first = 0,
                              int last = 1 << 30) {
  int idx = 0;
  auto want = [&]() { const bool r = idx >= first && idx < last; ++idx; return r; };
  const int n = a.n, dh = a.dh, m = a.m, C = a.C;
  const int k = n / C;
  const int64_t md = (int64_t)m * dh, io = (int64_t)bh0 * n * dh;
  const LactWs L = lact_layout<T>(BH, dh, m, C);
  T* Hh = (T*)(wsg + L.Hh);
  T* A = (T*)(wsg + L.A);
  T* U = (T*)(wsg + L.U);
  T* R = (T*)(wsg + L.R);
  T* dA = (T*)(wsg + L.dA);
  T* dU = (T*)(wsg + L.dU);
  T* W1s = (T*)(wsg + L.W1s);
  T* W3s = (T*)(wsg + L.W3s);
  T* W2s = (T*)(wsg + L.W2s);
  float* part = (float*)(wsg + L.part);
  T* mX0 = (T*)(wsg + L.mX0);
  T* mX1 = (T*)(wsg + L.mX1);
  T* mA = (T*)(wsg + L.mA);
  T* mB = (T*)(wsg + L.mB);
  float* mnorm = (float*)(wsg + L.mnorm);
  const int mr = m < dh ? m : dh, mc = m < dh ? dh : m;     // Muon's wide orientation [mr, mc]
  const T* q = (const T*)a.q + io;
  const T* kk = (const T*)a.k + io;
  const T* v = (const T*)a.v + io;
  T* O = (T*)a.O + io;
  float* W1f = a.W1f + bh0 * md;
  float* W3f = a.W3f + bh0 * md;
  float* W2f = a.W2f + bh0 * md;
  const float* eta_tok = a.eta_tok != nullptr ? a.eta_tok + (int64_t)bh0 * n : nullptr;
  const dim3 ew((unsigned)cdiv(md / 4, 256), (unsigned)(BH * 3));
  hipError_t e;

  if (want()) k_lact_init<T><<<ew, 256, 0, s>>>((const T*)a.W1, (const T*)a.W3, (const T*)a.W2, W1f, W3f, W2f, W1s, W3s, W2s,
                                    bh0, a.H, dh, m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // kept states: slot c of row bh at keep + ((c B H + bh0 + bh) 3 + w) m dh
  auto keep_slot = [&](int c) -> hipError_t {
    if (a.keep == nullptr) return hipSuccess;
    T* dst = (T*)a.keep + ((int64_t)c * a.B * a.H + bh0) * 3 * md;
    k_lact_keep<T><<<ew, 256, 0, s>>>(W1s, W3s, W2s, dst, md);
    return hipGetLastError();
  };
  if ((e = keep_slot(0)) != hipSuccess) return e;
  if (n == 0) return hipSuccess;

  const int kslice = (int)(cdiv(cdiv(C, kSplit), 64) * 64);
  const bool upd_first = a.order == 0;
  const int steps = upd_first ? k + 1 : k;
  for (int c = 0; c < steps; ++c) {
    StepRows sr;
    if (upd_first) {
      sr.qc = c - 1;
      sr.kc = c;
      sr.nq = c >= 1 ? C : 0;
      sr.nk = c < k ? C : 0;
    } else {
      sr.qc = sr.kc = c;
      sr.nq = sr.nk = C;
    }
    if (sr.nk > 0 && a.update_mask != nullptr && a.update_mask[sr.kc] == 0) sr.nk = 0;   // applied only
    if (a.keys_only) sr.nq = 0;                                   // the backward's recompute: states only
    // a chunk that does not update passes the state on unchanged: its kept slot is the same state
    const bool passes = sr.nk == 0 && sr.kc < k;
    if (sr.nq == 0 && sr.nk == 0) {
      if (passes && (e = keep_slot(sr.kc + 1)) != hipSuccess) return e;
      continue;
    }
    const int tq1 = (int)(cdiv(sr.nq, Wide::BQ) + cdiv(sr.nk, Wide::BQ));
    const int64_t hpart = (int64_t)BH * C * m;
    if (want())
      k_lact_fwd1<T><<<(unsigned)(cdiv(m, Wide::BP / 2) * tq1 * BH), Wide::NT, 0, s>>>(q, kk, W1s, W3s, Hh, A, U, BH,
                                                                                     n, dh, m, C, sr, md, hpart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int tq2 = (int)(cdiv(sr.nq, Wide::BQ) + cdiv(sr.nk, Wide::BQ));
    if (want())
      k_lact_fwd2<T><<<(unsigned)(cdiv(dh, Wide::BP) * tq2 * BH), Wide::NT, 0, s>>>(Hh, W2s, v, O, R, BH, n, dh, m, C,
                                                                                 sr, eta_tok, a.loss_dot, md, hpart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (sr.nk == 0) {
      if (passes && (e = keep_slot(sr.kc + 1)) != hipSuccess) return e;
      continue;
    }
    if (want()) k_lact_dh<T><<<(unsigned)(cdiv(m, Wide::BP) * cdiv(sr.nk, Wide::BQ) * BH), Wide::NT, 0, s>>>(
        R, W2s, A, U, dA, dU, BH, dh, m, C, sr.nk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t tg = (2 * cdiv(dh, Wide::BP) * cdiv(m, Wide::BQ) + cdiv(m, Wide::BP) * cdiv(dh, Wide::BQ)) *
                       (int64_t)kSplit * BH;
    if (want()) k_lact_grad<T><<<(unsigned)tg, Wide::NT, 0, s>>>(kk, dA, dU, Hh, R, part, BH, n, dh, m, C, sr.kc, sr.nk, kslice);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.muon) {
      const dim3 nsr((unsigned)(cdiv(mr, Half::BP) * cdiv(mr, Half::BQ)), (unsigned)(3 * BH));
      const dim3 nsx((unsigned)(cdiv(mc, Half::BP) * cdiv(mr, Half::BQ)), (unsigned)(3 * BH));
      if (want()) k_muon_norm<<<dim3(kMuonNormBlocks, (unsigned)(3 * BH)), 256, 0, s>>>(part, mnorm, BH, md);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (want())
        k_muon_prep<T><<<dim3((unsigned)cdiv(md, 256), (unsigned)(3 * BH)), 256, 0, s>>>(part, mnorm, mX0, BH, dh, m);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      T* xs = mX0;
      T* xn = mX1;
      for (int it = 0; it < kMuonSteps; ++it) {
        if (want()) k_ns_gemm<T, 0><<<nsr, Half::NT, 0, s>>>(xs, nullptr, nullptr, mA, mr, mc);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (want()) k_ns_gemm<T, 1><<<nsr, Half::NT, 0, s>>>(nullptr, mA, nullptr, mB, mr, mc);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (want()) k_ns_gemm<T, 2><<<nsx, Half::NT, 0, s>>>(xs, nullptr, mB, xn, mr, mc);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        T* t = xs;
        xs = xn;
        xn = t;
      }
      if (want()) k_lact_update_muon<T><<<ew, 256, 0, s>>>(xs, W1f, W3f, W2f, W1s, W3s, W2s, dh, m, a.eta);
    } else if (want()) {
      k_lact_update<T><<<ew, 256, 0, s>>>(part, W1f, W3f, W2f, W1s, W3s, W2s, BH, dh, m, a.eta);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.weight_norm && want())
      k_lact_wnorm<T><<<dim3((unsigned)cdiv(dh > m ? dh : m, 4), (unsigned)(BH * 3)), 256, 0, s>>>(
          W1f, W3f, W2f, W1s, W3s, W2s, dh, m);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = keep_slot(sr.kc + 1)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// The backward's passes over one chunk's rows X (keys or queries of chunk c)
// with the states at W (row bh's W1, W3, W2 at W + bh wsb + 0, m dh, 2 m dh):
// A, U and Hh = silu(A) U (all [BH, C, m]); and R = Hh W2^T - v (squared
// error, rounded once) [BH, C, dh].
template <typename T>
hipError_t launch_lact_gate_pass(const T* X, const T* W, int64_t wsb, T* A, T* U, T* Hh, int BH, int n, int dh,
                                 int m, int C, int c, hipStream_t s) {
  const StepRows sr{0, C, 0, c};
  const int64_t md = (int64_t)m * dh;
  k_lact_fwd1<T><<<(unsigned)(cdiv(m, Wide::BP / 2) * cdiv(C, Wide::BQ) * BH), Wide::NT, 0, s>>>(
      X, X, W, W + md, Hh, A, U, BH, n, dh, m, C, sr, wsb, 0);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_lact_residual_pass(const T* Hh, const T* W, int64_t wsb, const T* v, T* R, int BH, int n, int dh,
                                     int m, int C, int c, hipStream_t s) {
  const StepRows sr{0, C, 0, c};
  k_lact_fwd2<T><<<(unsigned)(cdiv(dh, Wide::BP) * cdiv(C, Wide::BQ) * BH), Wide::NT, 0, s>>>(
      Hh, W + 2 * (int64_t)m * dh, v, nullptr, R, BH, n, dh, m, C, sr, nullptr, 0, wsb, 0);
  return hipGetLastError();
}

// Without a side stream the rows run as one chain on s.  With one, group 0
// runs on s and group 1 on the side stream, between the fork event recorded
// on s (after group 0's lead) and the join event that s waits for, so that the
// whole call is ordered on s like a single launch.  The side stream and both
// events belong to the caller.
template <typename T>
hipError_t launch_lact(const LactArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  const int G = a.side == nullptr ? 1 : (BH < kGroups ? BH : kGroups);
  if (G == 1) return enqueue_lact_group<T>(a, 0, BH, a.ws, s);
  static_assert(kGroups == 2, "one side stream");
  const int rows0 = group_rows(BH, G, 0);
  const size_t off1 = lact_layout<T>(rows0, a.dh, a.m, a.C).total;
  hipError_t e = enqueue_lact_group<T>(a, 0, rows0, a.ws, s, 0, kLead);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(a.fork, s)) != hipSuccess) return e;
  e = hipStreamWaitEvent(a.side, a.fork, 0);
  if (e == hipSuccess) e = enqueue_lact_group<T>(a, rows0, group_rows(BH, G, 1), a.ws + off1, a.side);
  hipError_t first = e;
  // the join is recorded even after an error, so that s never runs ahead of
  // work already enqueued on the side stream
  e = hipEventRecord(a.join, a.side);
  if (first == hipSuccess) first = e;
  e = enqueue_lact_group<T>(a, 0, rows0, a.ws, s, kLead);
  if (first == hipSuccess) first = e;
  e = hipStreamWaitEvent(s, a.join, 0);
  if (first == hipSuccess) first = e;
  return first;
}

template size_t lact_workspace_bytes<float>(int, int, int, int, int, int);
template size_t lact_workspace_bytes<bf16>(int, int, int, int, int, int);
template hipError_t launch_lact<float>(const LactArgs&, hipStream_t);
template hipError_t launch_lact<bf16>(const LactArgs&, hipStream_t);
#define TTT_LACT_PASSES(T)                                                                                          \
  template hipError_t launch_lact_gate_pass<T>(const T*, const T*, int64_t, T*, T*, T*, int, int, int, int, int,  \
                                               int, hipStream_t);                                                 \
  template hipError_t launch_lact_residual_pass<T>(const T*, const T*, int64_t, const T*, T*, int, int, int, int, \
                                                   int, int, hipStream_t);
TTT_LACT_PASSES(float)
TTT_LACT_PASSES(bf16)
#undef TTT_LACT_PASSES

}  // namespace ttt
