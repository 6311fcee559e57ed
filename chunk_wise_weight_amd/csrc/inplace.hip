// In-Place TTT kernels for gfx950: the producers of Z and V^, the dot-objective
// deltas / prefix scan / fused update-scan, the apply, and the MSE chunk scan.
// Layer semantics: review of "In-Place Test-Time Training", Method §1-§3.
//
// Activation layouts (B batch rows, n tokens, d = d_model, f = d_ff):
//   Z  [B, n, f]   read by the apply (K = f contiguous)
//   Zt [B, f, n]   read by the updates (K = tokens contiguous)
//   Vt [B, d, n]   the target V^, transposed, read by the updates
// so that every contraction reads both operands K-contiguously.
#include <cstdlib>
#include <type_traits>

#include "gemm.hpp"
#include "launch.hpp"

namespace ttt {

// Packed documents: docs [B, k] (may be null) flags the chunks that start a new
// document in their batch row; chunk 0 always starts one unless the call
// resumes its rows (cont), when only a flag does.  At a document start the
// state starts again from W_down0 and the convolution from zeros, so that
// nothing of the previous document reaches it (Method §3, document boundaries).
__device__ __forceinline__ bool doc_start(const uint8_t* __restrict__ docs, int64_t b, int k, int c,
                                          bool cont = false) {
  if (c == 0 && !cont) return true;
  return docs != nullptr && docs[b * k + c] != 0;
}

// Update mask [B, k] (device; null: every chunk updates).  A chunk whose flag
// is zero is applied but leaves the state as it found it; its target (dot
// objective) or residual (MSE) is multiplied by zero instead, so the update's
// accumulation adds exact zeros.
__device__ __forceinline__ float update_flag(const uint8_t* __restrict__ umask, int64_t b, int k, int c) {
  return umask == nullptr || umask[b * k + c] != 0 ? 1.0f : 0.0f;
}


template <typename T> constexpr int esz() { return (int)sizeof(T); }

// ------------------------------------------------------------------ conv, transpose

// (the backward of the convolution follows k_conv below)

// Y = CausalDepthwiseConv1D_KW(X0) (eq. (5) with the causal padding of §3):
// Y[t, ch] = sum_j conv_w[ch, j] * X0[t - (KW-1) + j, ch], zero before the
// sequence start.  One thread: RW consecutive rows x one 16-byte channel
// chunk, reading each of the RW + KW - 1 input rows it needs once (a sliding
// window; RW divides n, so a thread's rows never straddle a batch row).
constexpr int kConvRows = 8;
static_assert(kConvRows == kConvBwdRows, "the convolution's backward takes the forward's row groups");
// FWD: the forward-looking in-chunk reading -- tap j multiplies the token j
// steps ahead, and tokens past the chunk's end are zero (the review's
// next-token example, Method §2); else tap KW - 1 is the current token.
template <typename T, int KW, bool FWD>
__global__ __launch_bounds__(256) void k_conv(const T* __restrict__ X0, const T* __restrict__ cw, T* __restrict__ Y,
                                              int64_t rows, int n, int d, const uint8_t* __restrict__ docs, int C_,
                                              const T* __restrict__ halo) {
  constexpr int V = Vec<T>::V, RW = kConvRows, NIN = RW + KW - 1;
  const int nchunk = d / V;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (rows / RW) * nchunk) return;
  const int ch = (int)(gid % nchunk) * V;
  const int64_t r0 = (gid / nchunk) * RW;
  const int pos0 = (int)(r0 % n);                  // position of row r0 in its sequence
  // first row of its document, and the end of its chunk: the thread's rows lie
  // in one chunk (C_ % 8 == 0)
  const int lo = doc_start(docs, r0 / n, n / C_, pos0 / C_) ? (pos0 / C_) * C_ : 0;
  const int hi = (pos0 / C_ + 1) * C_;
  // a resumed row reads the previous call's last KW - 1 rows (halo [B, KW - 1, d])
  // before its first token, unless a document starts there
  const bool use_halo = !FWD && halo != nullptr && pos0 == 0 && !doc_start(docs, r0 / n, n / C_, 0, true);
  const T* hrow = use_halo ? halo + ((r0 / n) * (KW - 1)) * (int64_t)d + ch : nullptr;
  float w[V][KW];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(cw + (int64_t)ch * KW);
#pragma unroll
    for (int c = 0; c < KW; ++c) {   // V * KW elements = KW chunks of 16 bytes
      const u32x4 x = src[c];
      float fv[V];
      if constexpr (sizeof(T) == 2) unpack8(x, fv);
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) fv[e] = __uint_as_float(x[e]);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) w[(c * V + e) / KW][(c * V + e) % KW] = fv[e];
    }
  }
  // input row i of the window is X0 row r0 - (KW - 1) + i (FWD: r0 + i); rows
  // before the document start (FWD: from the chunk's end on) are zero
  u32x4 in[NIN];
  const T* base = X0 + (r0 - (FWD ? 0 : KW - 1)) * d + ch;
#pragma unroll
  for (int i = 0; i < NIN; ++i) {
    const bool live = FWD ? (i < RW || pos0 + i < hi) : (i >= KW - 1 || pos0 + i - (KW - 1) >= lo);
    if (live) in[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)i * d);
    else if (use_halo && i < KW - 1) in[i] = *reinterpret_cast<const u32x4*>(hrow + (int64_t)i * d);
    else in[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float y[V];
#pragma unroll
    for (int v = 0; v < V; ++v) y[v] = 0.f;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      float xf[V];
      if constexpr (sizeof(T) == 2) unpack8(in[r + j], xf);
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) xf[e] = __uint_as_float(in[r + j][e]);
      }
#pragma unroll
      for (int v = 0; v < V; ++v) y[v] = fmaf(w[v][j], xf[v], y[v]);
    }
    u32x4 o;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack2_bf16(y[2 * e], y[2 * e + 1]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(y[e]);
    }
    *reinterpret_cast<u32x4*>(Y + (r0 + r) * d + ch) = o;
  }
}

// Backward of the causal convolution of k_conv:
// dX0[s, ch] = sum_j conv_w[ch, j] dY[s + (KW-1) - j, ch], rows past the end of
// s's document zero; and dconv_w[ch, j] = sum_t dY[t, ch] X0[t - (KW-1) + j, ch],
// rows before the start of t's document zero -- or, for a resumed row's first
// document, the halo's rows (halo [B, KW-1, d]), whose gradient
// dhalo[b, h, ch] = sum_{j <= h} conv_w[ch, j] dY[h - j, ch] the group holding
// the row's first token writes (zero where chunk 0 starts a document; dhalo
// may be null).  Documents start at chunk boundaries and KW - 1 < C_, so a
// group's windows reach at most the next chunk (dY) or the previous one (X0).
// One thread: one 16-byte channel chunk over kConvBwdGroups groups of
// kConvRows rows (each group inside one batch row), writing its share of
// dconv_w to part [blocks, d, KW] (fp32), which a row sum then reduces.
template <typename T, int KW, bool FWD>
__global__ __launch_bounds__(256) void k_conv_bwd(const T* __restrict__ X0, const T* __restrict__ cw,
                                                  const T* __restrict__ dY, T* __restrict__ dX0,
                                                  float* __restrict__ part, int64_t rows, int n, int d,
                                                  const uint8_t* __restrict__ docs, int C_,
                                                  const T* __restrict__ halo, T* __restrict__ dhalo) {
  constexpr int V = Vec<T>::V, RW = kConvRows, NIN = RW + KW - 1;
  const int nchunk = d / V;
  const int64_t ngroups = rows / RW;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= conv_bwd_partials(rows) * nchunk) return;
  const int ch = (int)(gid % nchunk) * V;
  const int64_t pb = gid / nchunk;
  float w[V][KW], gw[V][KW];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(cw + (int64_t)ch * KW);
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      const u32x4 x = src[c];
      float fv[V];
      if constexpr (sizeof(T) == 2) unpack8(x, fv);
      else {
#pragma unroll
        for (int e = 0; e < 4; ++e) fv[e] = __uint_as_float(x[e]);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) w[(c * V + e) / KW][(c * V + e) % KW] = fv[e];
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int j = 0; j < KW; ++j) gw[v][j] = 0.f;
  auto unpack = [](u32x4 x, float* o) {
    if constexpr (sizeof(T) == 2) unpack8(x, o);
    else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(x[e]);
    }
  };
  for (int gi = 0; gi < kConvBwdGroups; ++gi) {
    const int64_t grp = pb * kConvBwdGroups + gi;
    if (grp >= ngroups) break;
    const int64_t r0 = grp * RW;
    const int pos0 = (int)(r0 % n);
    // this group's chunk and document bounds: lo = its document's first row if the chunk starts one (else the
    // window never reaches back past the document's start); hi = the first row of the next document if the next
    // chunk starts one (else the sequence end, or further)
    const int64_t row = r0 / n;
    const int kc = n / C_, c = pos0 / C_;
    const int lo = doc_start(docs, row, kc, c) ? c * C_ : 0;
    const int hi = c + 1 < kc && docs != nullptr && docs[row * kc + c + 1] != 0 ? (c + 1) * C_ : n;
    // causal: gy[i] = dY row r0 + i (zero from hi on), xs[i] = X0 row r0 - (KW-1) + i (zero before lo).
    // FWD (Y[t] = sum_j w_j X0[t + j] inside t's chunk): gy[i] = dY row r0 - (KW-1) + i (zero before the
    // chunk's first row), xs[i] = X0 row r0 + i (zero from the next chunk on); a window never leaves the chunk,
    // so documents, which start at chunk boundaries, need nothing more.
    // a resumed row's first group reads the halo before its first token (never with FWD)
    const bool use_halo = !FWD && halo != nullptr && pos0 == 0 && !doc_start(docs, row, kc, 0, true);
    const T* hrow = use_halo ? halo + (row * (KW - 1)) * (int64_t)d + ch : nullptr;
    u32x4 gy[NIN], xs[NIN];
#pragma unroll
    for (int i = 0; i < NIN; ++i) {
      if constexpr (FWD) {
        gy[i] = pos0 + i - (KW - 1) >= c * C_ ? *reinterpret_cast<const u32x4*>(dY + (r0 + i - (KW - 1)) * d + ch)
                                              : u32x4{0u, 0u, 0u, 0u};
        xs[i] = pos0 + i < (c + 1) * C_ ? *reinterpret_cast<const u32x4*>(X0 + (r0 + i) * d + ch)
                                        : u32x4{0u, 0u, 0u, 0u};
      } else {
        gy[i] = pos0 + i < hi ? *reinterpret_cast<const u32x4*>(dY + (r0 + i) * d + ch) : u32x4{0u, 0u, 0u, 0u};
        xs[i] = pos0 + i - (KW - 1) >= lo ? *reinterpret_cast<const u32x4*>(X0 + (r0 + i - (KW - 1)) * d + ch)
                : use_halo && i < KW - 1  ? *reinterpret_cast<const u32x4*>(hrow + (int64_t)i * d)
                                          : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (KW > 1 && dhalo != nullptr && pos0 == 0) {
      // halo row h sits at position h - (KW-1): output t reads it through tap j = h - t
#pragma unroll
      for (int h = 0; h < KW - 1; ++h) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = 0.f;
        if (use_halo) {
#pragma unroll
          for (int j = 0; j <= h; ++j) {
            float y[V];
            unpack(gy[h - j], y);
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = fmaf(w[v][j], y[v], o[v]);
          }
        }
        u32x4 out;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = pack2_bf16(o[2 * e], o[2 * e + 1]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(o[e]);
        }
        *reinterpret_cast<u32x4*>(dhalo + (row * (KW - 1) + h) * (int64_t)d + ch) = out;
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      float o[V], g[V];
#pragma unroll
      for (int v = 0; v < V; ++v) o[v] = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        float y[V], x[V];
        unpack(gy[r + KW - 1 - j], y);
        unpack(xs[r + j], x);
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = fmaf(w[v][j], y[v], o[v]);
        if (j == 0) unpack(gy[FWD ? r + KW - 1 : r], g);       // dY row r0 + r
#pragma unroll
        for (int v = 0; v < V; ++v) gw[v][j] = fmaf(g[v], x[v], gw[v][j]);
      }
      u32x4 out;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack2_bf16(o[2 * e], o[2 * e + 1]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(o[e]);
      }
      *reinterpret_cast<u32x4*>(dX0 + (r0 + r) * d + ch) = out;
    }
  }
  float* pp = part + (pb * d + ch) * KW;
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int j = 0; j < KW; ++j) pp[v * KW + j] = gw[v][j];
}

// dst[b][c][r] = scale * src[b][r][c] for an R x C matrix per batch entry (64 x 64 tiles).
// rev > 0: the rows come in blocks of rev (chunks) whose order is reversed in
// dst, i.e. r lands at column (R / rev - 1 - r / rev) rev + r % rev.
// umask (with chunk > 0): the rows are tokens of chunks of `chunk` rows, and
// rows of chunks whose update flag is zero are scaled by zero.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, T* __restrict__ dst, int R, int C,
                                                   float scale, int rev, const uint8_t* __restrict__ umask,
                                                   int chunk) {
  __shared__ T tile[64][65];
  const int64_t b = blockIdx.y;
  const int tc = (C + 63) / 64;
  const int r0 = (int)(blockIdx.x / tc) * 64, c0 = (int)(blockIdx.x % tc) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const T* s = src + b * (int64_t)R * C;
  T* o = dst + b * (int64_t)R * C;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = s[(int64_t)r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    const int rr = rev > 0 ? (R / rev - 1 - r / rev) * rev + r % rev : r;
    const float sc = umask != nullptr && r < R ? scale * update_flag(umask, blockIdx.y, R / chunk, r / chunk) : scale;
    if (c < C && r < R) o[(int64_t)c * R + rr] = sc == 1.0f ? tile[tx][i] : from_f32<T>(sc * to_f32(tile[tx][i]));
  }
}

// ------------------------------------------------------------------ producers

// Z = silu(H W_gate^T) * (H W_up^T)  (eq. (2)).  P = tokens, Q = gate and up
// rows in alternating 32-row blocks, so a lane holds the gate and the up value
// of one output column in Q blocks 0 and 1, for 4 consecutive tokens.
// Writes Zt[b, j, t..t+3] (packed) and, if Z is given, Z[t + e, j].
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_produce_z(const T* __restrict__ H, const T* __restrict__ Wg, const T* __restrict__ Wu,
                                       T* __restrict__ Z, T* __restrict__ Zt, int64_t rows, int n, int d, int f) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (int)((rows + G::BP - 1) / G::BP), TQ = (f + G::BQ / 2 - 1) / (G::BQ / 2);
  int tp, tq;
  // groups of 6 token tiles sweep every weight tile: the weights (a few
  // hundred MB at most) stay in the last-level cache while the tokens stream
  // from HBM once, not once per group of weight tiles; an XCD's 32 concurrent
  // tiles are then about 6 token x 5 weight tiles, 11 operand row blocks per K
  // step rather than 12 for 8 x 4 (produce_z 10.64 -> 10.55 ms on one box,
  // 10.60 -> 10.32 on another)
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), TQ, TP, 6, tq, tp);
  const int64_t t0 = (int64_t)tp * G::BP;
  const int j0 = tq * (G::BQ / 2);
  const uint64_t ldb = (uint64_t)d * esz<T>();

  DmaOp<G::NW, G::BP> op;
  op.init(H + t0 * d, nullptr, (int)min<int64_t>(G::BP, rows - t0), ldb, (unsigned)ldb);
  DmaOp<G::NW, G::BQ, true> oq;
  oq.init(Wg + (int64_t)j0 * d, Wu + (int64_t)j0 * d, min(G::BQ / 2, f - j0), ldb, (unsigned)ldb);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  // Each wave's 64 Q rows are 32 W_gate rows (blocks 0, 1) then the same 32
  // W_up rows (blocks 2, 3): block jj pairs with block jj + 2.  Z replaces the
  // gate value in place.
  static_assert(G::NQB == 4 && G::BM == 16 && G::GPB == 1, "two gate/up block pairs per wave");
#pragma unroll
  for (int i = 0; i < G::NPB; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][jj][e] = silu_f(acc[i][jj][e]) * acc[i][jj + 2][e];
  const int jl = (wave_id() % G::WQ) * 32 + (lane_id() & 15);      // local column of block jj = 0
  const int jn = min(G::BQ / 2, f - j0);
  const int tn = (int)min<int64_t>(G::BP, rows - t0);

  // Zt [b, j, t]: staged as [128 columns][256 tokens]; a 16-byte piece holds
  // 8 (bf16) or 4 (fp32) tokens, which never straddle a batch row (n % 8 == 0).
  if (Zt != nullptr) {
    const Staged<T, G::BP> st{smem};
#pragma unroll
    for (int i = 0; i < G::NPB; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        st.put4(jl + 16 * jj, G::acc_p(i, 0), acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]);
    __syncthreads();
    st.template flush<G::NT, G::BQ / 2, false, 0>(jn, [&](int r, int col) -> T* {
      if (col >= tn) return nullptr;
      const int64_t tok = t0 + col, b = tok / n;
      return Zt + (b * f + j0 + r) * (int64_t)n + (tok - b * n);
    });
    __syncthreads();
  }
  // Z [t, j]: staged as [256 tokens][128 columns]
  if (Z != nullptr) {
    const Staged<T, G::BQ / 2> sz{smem};
#pragma unroll
    for (int i = 0; i < G::NPB; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) sz.put1(G::acc_p(i, 0) + e, jl + 16 * jj, acc[i][jj][e]);
    __syncthreads();
    sz.template flush<G::NT, G::BP, false, 0>(tn, [&](int r, int col) -> T* {
      return col < jn ? Z + (t0 + r) * f + j0 + col : nullptr;
    });
  }
}

// Backward of the producer (eq. (2)) given dZ [rows, f]: the K loop recomputes
// A = H W_gate^T and U = H W_up^T exactly as k_produce_z does, and the epilogue
// forms dA = dZ U silu'(A) and dU = dZ silu(A), silu'(a) = s (1 + a (1 - s))
// with s the logistic function, written as G [rows, 2f]: dA in columns
// 0 .. f - 1, dU in f .. 2f - 1 (one matrix, so that one token contraction
// gives both weight gradients).  dZ is read element by element: a lane's four
// tokens at one column, 32 bytes of a row per 16 lanes.
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_produce_z_bwd(const T* __restrict__ H, const T* __restrict__ Wg,
                                           const T* __restrict__ Wu, const T* __restrict__ dZ, T* __restrict__ Gout,
                                           int64_t rows, int n, int d, int f) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (int)((rows + G::BP - 1) / G::BP), TQ = (f + G::BQ / 2 - 1) / (G::BQ / 2);
  int tp, tq;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), TQ, TP, 6, tq, tp);   // as k_produce_z
  const int64_t t0 = (int64_t)tp * G::BP;
  const int j0 = tq * (G::BQ / 2);
  const uint64_t ldb = (uint64_t)d * esz<T>();

  DmaOp<G::NW, G::BP> op;
  op.init(H + t0 * d, nullptr, (int)min<int64_t>(G::BP, rows - t0), ldb, (unsigned)ldb);
  DmaOp<G::NW, G::BQ, true> oq;
  oq.init(Wg + (int64_t)j0 * d, Wu + (int64_t)j0 * d, min(G::BQ / 2, f - j0), ldb, (unsigned)ldb);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  // block jj holds A, block jj + 2 the matching U (the layout of k_produce_z)
  static_assert(G::NQB == 4 && G::BM == 16 && G::GPB == 1, "two gate/up block pairs per wave");
  const int jl = (wave_id() % G::WQ) * 32 + (lane_id() & 15);
  const int jn = min(G::BQ / 2, f - j0);
  const int tn = (int)min<int64_t>(G::BP, rows - t0);
  const int64_t ldg = 2 * (int64_t)f;
  // bf16: the dZ tile [256 tokens][128 columns] (64 KB) comes into the first
  // half of the LDS with 16-byte loads, dA is staged in the second half while
  // it is read, and dU then replaces it.  fp32 (128 KB tiles): dZ is read from
  // memory element by element and the two results share the LDS in turn.
  constexpr bool kStageDz = sizeof(T) == 2;
  constexpr int kHalf = G::BP * (G::BQ / 2) * (int)sizeof(T);
  constexpr int kFlushBatch = sizeof(T) == 2 ? 8 : 0;          // fp32: no registers to spare
  const Staged<T, G::BQ / 2> sdz{smem}, sda{smem + (kStageDz ? kHalf : 0)};
  if constexpr (kStageDz) {
    constexpr int PPR = (G::BQ / 2) * (int)sizeof(T) / 16;          // 16-byte pieces per row
    for (int idx = threadIdx.x; idx < tn * PPR; idx += G::NT) {
      const int r = idx / PPR, c = (idx - r * PPR) * (16 / (int)sizeof(T));
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (c < jn) v = *reinterpret_cast<const u32x4*>(dZ + (t0 + r) * f + j0 + c);
      *reinterpret_cast<u32x4*>(smem + sdz.off(r, c)) = v;
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < G::NPB; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tr = G::acc_p(i, 0) + e, jc = jl + 16 * jj;
        float dz;
        if constexpr (kStageDz) dz = tr < tn ? to_f32(*reinterpret_cast<const T*>(smem + sdz.off(tr, jc))) : 0.f;
        else dz = (tr < tn && jc < jn) ? to_f32(dZ[(t0 + tr) * f + j0 + jc]) : 0.f;
        const float a = acc[i][jj][e], u = acc[i][jj + 2][e], sg = sigmoid_f(a);
        const float da = dz * u * sg * (1.0f + a * (1.0f - sg));
        acc[i][jj + 2][e] = dz * a * sg;                 // dU
        if constexpr (kStageDz) sda.put1(tr, jc, da);
        else acc[i][jj][e] = da;
      }
  if constexpr (!kStageDz) {
#pragma unroll
    for (int i = 0; i < G::NPB; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) sda.put1(G::acc_p(i, 0) + e, jl + 16 * jj, acc[i][jj][e]);
  }
  __syncthreads();
  // dA out as whole rows of G; then dU staged over the dZ tile (read by all waves before the barrier above)
  sda.template flush<G::NT, G::BP, false, kFlushBatch>(tn, [&](int r, int col) -> T* {
    return col < jn ? Gout + (t0 + r) * ldg + j0 + col : nullptr;
  });
  if constexpr (!kStageDz) __syncthreads();
#pragma unroll
  for (int i = 0; i < G::NPB; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 4; ++e) sdz.put1(G::acc_p(i, 0) + e, jl + 16 * jj, acc[i][jj + 2][e]);
  __syncthreads();
  sdz.template flush<G::NT, G::BP, false, kFlushBatch>(tn, [&](int r, int col) -> T* {
    return col < jn ? Gout + (t0 + r) * ldg + f + j0 + col : nullptr;
  });
}

// Vt = scale * (Y W_target)^T with WtT = W_target^T [d_out, d_in].  P = tokens,
// Q = output channels; writes Vt[b, o, t..t+3].
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_produce_vhat(const T* __restrict__ Y, const T* __restrict__ WtT, T* __restrict__ Vt,
                                          int64_t rows, int n, int d, float scale, const uint8_t* __restrict__ umask,
                                          int C_) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (int)((rows + G::BP - 1) / G::BP), TQ = (d + G::BQ - 1) / G::BQ;
  int tp, tq;
  // groups of 8 token tiles sweep every weight tile: the weights (a few
  // hundred MB at most) stay in the last-level cache while the tokens stream
  // from HBM once, not once per group of weight tiles
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), TQ, TP, 8, tq, tp);
  const int64_t t0 = (int64_t)tp * G::BP;
  const int o0 = tq * G::BQ;
  const uint64_t ldb = (uint64_t)d * esz<T>();

  DmaOp<G::NW, G::BP> op;
  DmaOp<G::NW, G::BQ> oq;
  op.init(Y + t0 * d, nullptr, (int)min<int64_t>(G::BP, rows - t0), ldb, (unsigned)ldb);
  oq.init(WtT + (int64_t)o0 * d, nullptr, min(G::BQ, d - o0), ldb, (unsigned)ldb);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  // Vt [b, o, t]: staged as [output channel][token] in as many passes as the
  // stage area needs (one for bf16, two for fp32).  A lane's four tokens lie in
  // one chunk of one batch row (n and C_ are multiples of 8), so they share
  // one update flag.
  const int tn = (int)min<int64_t>(G::BP, rows - t0);
  float sc[G::NPB];
#pragma unroll
  for (int i = 0; i < G::NPB; ++i) {
    const int64_t tok = min<int64_t>(t0 + G::acc_p(i, 0), rows - 1), b = tok / n;
    sc[i] = umask != nullptr ? scale * update_flag(umask, b, n / C_, (int)(tok - b * n) / C_) : scale;
  }
  constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(T) + G::Smem - 1) / G::Smem, RPP = G::BQ / PASSES;
  const Staged<T, G::BP> st{smem};
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int j = 0; j < G::NQB; ++j) {
      const int q = G::acc_q(j) - ps * RPP;
      if (q < 0 || q >= RPP) continue;
#pragma unroll
      for (int i = 0; i < G::NPB; ++i)
        st.put4(q, G::acc_p(i, 0), sc[i] * acc[i][j][0], sc[i] * acc[i][j][1], sc[i] * acc[i][j][2],
                sc[i] * acc[i][j][3]);
    }
    __syncthreads();
    st.template flush<G::NT, RPP, false, 0>(RPP, [&](int r, int col) -> T* {
      const int o = o0 + ps * RPP + r;
      if (o >= d || col >= tn) return nullptr;
      const int64_t tok = t0 + col, b = tok / n;
      return Vt + (b * d + o) * (int64_t)n + (tok - b * n);
    });
    __syncthreads();
  }
}

// ------------------------------------------------------------------ dot objective

// Visit this lane's accumulator quads of a [d_model x d_ff] state tile (P = j,
// d_ff, contiguous; Q = i, d_model) with one row pointer per Q block plus
// small constant offsets.  fn(row_offset_elems, dj, ib, jb, g) is called for
// every quad inside the matrix.
template <class G, class Fn>
__device__ __forceinline__ void for_state_quads(int j0, int i0, int d, int f, Fn&& fn) {
  const bool full = j0 + G::BP <= f && i0 + G::BQ <= d;
  const int pl = G::acc_p(0, 0), ql = G::acc_q(0);
#pragma unroll
  for (int jb = 0; jb < G::NQB; ++jb) {
    const int i = i0 + ql + jb * G::BM;
    const int64_t rowoff = (int64_t)i * f + j0 + pl;
#pragma unroll
    for (int ib = 0; ib < G::NPB; ++ib) {
#pragma unroll
      for (int g = 0; g < G::GPB; ++g) {
        const int dj = ib * G::BM + g * 8;
        if (full || (i < d && j0 + pl + dj < f)) fn(rowoff, dj, ib, jb, g);
      }
      if (((ib + 1) * G::GPB) % 4 == 0) __builtin_amdgcn_sched_barrier(0);   // four quads at a time
    }
  }
}

template <class G, typename TO, class Acc>
__device__ __forceinline__ void store_state(const Acc& acc, TO* __restrict__ out, int j0, int i0, int d, int f) {
  for_state_quads<G>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
    const auto& blk = acc[ib][jb];
    store4(out + ro + dj, blk[4 * g], blk[4 * g + 1], blk[4 * g + 2], blk[4 * g + 3]);
  });
}

// store_state through LDS: the [d_model x d_ff] state tile (rows i = Q, columns
// j = P) is staged in BUFB bytes at buf, in as many passes over its rows as
// needed, and written out as whole 16-byte pieces along rows (non-temporal
// stores with STREAM).  Every wave must call it; it ends with a barrier.
// BATCH: the copy-out's LDS read batch (0: one piece at a time, for callers
// inside a K loop, whose accumulators stay live).
template <class G, int BUFB, typename TO, class Acc, bool STREAM = false, int BATCH = 0>
__device__ __forceinline__ void stage_state(const Acc& acc, TO* __restrict__ out, char* buf, int j0, int i0, int d,
                                            int f) {
  static_assert(G::GPB == 1, "one accumulator group per block");
  constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(TO) + BUFB - 1) / BUFB, RPP = G::BQ / PASSES;
  static_assert(RPP * PASSES == G::BQ && RPP * G::BP * (int)sizeof(TO) <= BUFB, "passes must tile the rows");
  const Staged<TO, G::BP> st{buf};
  const int jn = min(G::BP, f - j0), in_ = min(G::BQ, d - i0);
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int jb = 0; jb < G::NQB; ++jb) {
      const int q = G::acc_q(jb) - ps * RPP;
      if (q < 0 || q >= RPP) continue;
#pragma unroll
      for (int ib = 0; ib < G::NPB; ++ib)
        st.put4(q, G::acc_p(ib, 0), acc[ib][jb][0], acc[ib][jb][1], acc[ib][jb][2], acc[ib][jb][3]);
    }
    __syncthreads();
    auto dst = [&](int r, int col) -> TO* {
      return col < jn ? out + (int64_t)(i0 + ps * RPP + r) * f + j0 + col : nullptr;
    };
    st.template flush<G::NT, RPP, STREAM, BATCH>(max(0, min(RPP, in_ - ps * RPP)), dst);
    __syncthreads();
  }
}

// Per-chunk delta dW[b, c] = V^_c^T Z_c (Method §3, step 1), fp32 [B, k, d, f].
// P = d_ff rows of Zt, Q = d_model rows of Vt, K = the chunk's C tokens.
template <typename T>
TTT_GEMM_KERNEL(Wide) void k_chunk_delta(const T* __restrict__ Zt, const T* __restrict__ Vt, float* __restrict__ dW,
                                         int n, int d, int f, int C_) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (f + G::BP - 1) / G::BP, TQ = (d + G::BQ - 1) / G::BQ;
  const int per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bc = id / per;
  int tp, tq;
  grouped_tile(id - bc * per, TP, TQ, 4, tp, tq);
  const int k = n / C_;
  const int b = bc / k, c = bc - b * k;
  const int j0 = tp * G::BP, i0 = tq * G::BQ;
  const uint64_t ldb = (uint64_t)n * esz<T>();
  const unsigned kbytes = (unsigned)C_ * esz<T>();

  DmaOp<G::NW, G::BP> op;
  DmaOp<G::NW, G::BQ> oq;
  op.init(Zt + ((int64_t)b * f + j0) * n + (int64_t)c * C_, nullptr, min(G::BP, f - j0), ldb, kbytes);
  oq.init(Vt + ((int64_t)b * d + i0) * n + (int64_t)c * C_, nullptr, min(G::BQ, d - i0), ldb, kbytes);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((kbytes + 127) / 128), acc, smem, NoHook{});
  store_state<G>(acc, dW + (int64_t)bc * d * f, j0, i0, d, f);
}

// Exclusive prefix scan over chunks (Method §3, steps 2-3), four elements per
// thread: Wc[b, c] = W0 + eta * sum_{j<c} dW[b, j]; W_final = W0 + eta * sum_all.
// Inclusive (the update-then-apply order): Wc[b, c] = W0 + eta * sum_{j<=c}
// dW[b, j], the state after chunk c's own step.
template <typename T>
__global__ __launch_bounds__(256) void k_chunk_scan(const float* __restrict__ dW, const T* __restrict__ W0,
                                                    T* __restrict__ Wc, float* __restrict__ Wf, int k, int64_t df,
                                                    float eta, const uint8_t* __restrict__ docs,
                                                    const float* __restrict__ Winit, bool inclusive) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int b = blockIdx.y;
  if (e >= df) return;
  const f32x4 w0 = load4(W0 + e);
  // a resumed row (Winit) starts from its own state unless a document starts at chunk 0
  f32x4 base = (Winit != nullptr && !(k > 0 && doc_start(docs, b, k, 0, true))) ? load4(Winit + b * df + e) : w0;
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float* src = dW + (int64_t)b * k * df + e;
  T* dst = Wc + (int64_t)b * k * df + e;
  for (int c = 0; c < k; ++c) {
    if (c > 0 && doc_start(docs, b, k, c)) {
      s = (f32x4){0.f, 0.f, 0.f, 0.f};
      base = w0;
    }
    if (inclusive) s += load4(src + (int64_t)c * df);
    store4(dst + (int64_t)c * df, fmaf(eta, s[0], base[0]), fmaf(eta, s[1], base[1]), fmaf(eta, s[2], base[2]),
           fmaf(eta, s[3], base[3]));
    if (!inclusive) s += load4(src + (int64_t)c * df);
  }
  store4(Wf + (int64_t)b * df + e, fmaf(eta, s[0], base[0]), fmaf(eta, s[1], base[1]), fmaf(eta, s[2], base[2]),
         fmaf(eta, s[3], base[3]));
}

// Fused delta + scan.  The per-chunk delta does not depend on the state, so
// W_c = W_down0 + sum_{j<c} (eta V^_j)^T Z_j is the running value of ONE
// contraction over the tokens, read out at every chunk boundary: each
// workgroup owns one 256 x 256 tile of the state and runs its K loop in token
// order.  The target arrives pre-scaled by eta (eta times a delta is the delta
// of eta times the target), so the accumulator holds exactly the state.
//
// To fill the chip when the state has few tiles, the sequence is cut into S
// segments of k / S chunks that run side by side.  Segment 0 starts from
// W_down0 and writes the states W_c of its chunks in the operand dtype.  Two
// segments are chained (below).  With four, a later segment starts from zero
// and writes partial states to Wp (operand dtype) (chunks after its first) and
// its total to Tot[b, s - 1] -- except the last segment, whose total goes to
// W_final -- and k_scan_fixup then adds the earlier segments' totals.  With
// S = 1 the kernel alone produces every output.
// With packed documents the accumulator is set to W_down0 at every document
// start (a segment that begins with one starts from W_down0), so from there
// on a segment's states are absolute and the fix-up leaves them as they are.
// The states are written with non-temporal stores: the apply reads them back
// long after the caches would have dropped them.
//
// Chained segments (S = 2, `sync` given): the second segment does not leave
// its states partial.  Segment 0 publishes its end state (Tot, fp32) through a
// per-tile flag; segment 1 starts from zero and, at its first chunk boundary
// (one chunk of tokens into its K loop), waits for the flag and adds the end
// state to its accumulator, so that its states from there on are absolute and
// are rounded once.  The workgroups are ordered so that this never waits for
// long: each XCD runs its share of segment-0 tiles before the matching
// segment-1 tiles, and a segment-1 tile's partner is the segment-0 tile of the
// same state tile on the same XCD with a lower workgroup id, so the partner has
// been dispatched before it (it is running or done) and itself waits for
// nothing.  The wait is bounded (`wait` ticks of the 100 MHz wall clock,
// negative: do not wait); a tile whose partner has not published in time
// records that in its status word and keeps its states partial, and the
// fix-up kernel that follows completes those tiles alone (then rounding them
// twice).
// One thread polls the flag; its acquire (which invalidates this CU's vector
// cache, shared by the workgroup's waves) orders the workgroup's later reads
// of the partner's end state after the flag, and the barrier hands the result
// to every wave.
// Tile raster of the chained scan: groups of about 5 d_model tiles, each
// swept across the d_ff tiles, so that the 32 tiles an XCD runs at once (and
// the two half-rounds of first- and second-segment tiles it runs together)
// form compact blocks that share operand rows in its L2 (5 x 6 rather than
// 10 x 3 tiles).
__device__ __forceinline__ int chain_group(int TQ) {
  const int g = (TQ + 4) / 5;
  return (TQ + g - 1) / g;
}

__device__ __forceinline__ bool wait_published(const int* flag, long long wait, int* s_ok) {
  if (threadIdx.x == 0) {
    int v = 0;
    if (wait >= 0) {
      const long long t0 = wall_clock64();
      while ((v = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0 &&
             wall_clock64() - t0 < wait)
        __builtin_amdgcn_s_sleep(8);
    }
    if (v != 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_ok = v;
  }
  __syncthreads();
  return *s_ok != 0;
}

// INC (the update-then-apply order): the state written for chunk c is the one
// after its own step, W_{c+1}: at boundary c the accumulator is written as
// chunk c - 1's state before a document start at c resets it, and a segment
// ends by writing its last chunk's; no initial state is written.
template <typename T, bool INC = false>
struct SnapshotHook {
  T* Wc;              // [k, d, f] states of this batch row (segment 0, and chained segments)
  T* Wp;              // partial states of this batch row; chunk c at Wp + (c - kS) d f (later segments)
  const T* W0;        // W_down0, the state a packed document starts from
  const uint8_t* docs;  // document starts [B, k] or null
  int64_t b;
  int k, steps_per_chunk, c0, c1, kS, j0, i0, d, f;
  bool chain;          // chained segments: every state goes to Wc
  template <class A>
  __device__ __forceinline__ void reset(A& acc) const {
    for_state_quads<Wide>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
      const f32x4 w = load4(W0 + ro + dj);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ib][jb][4 * g + e] = w[e];
    });
  }
  // Chunk boundary c (the state before chunk c): a document start resets the
  // accumulator to W_down0, then the state is written (INC: the state is
  // written as chunk c - 1's first).
  template <class A>
  __device__ __forceinline__ void boundary(int c, A& acc, char* buf, bool doc) const {
    if (!INC && doc) reset(acc);     // a document starts at chunk c: its state is absolute
    const int64_t df = (int64_t)d * f;
    const int slot = INC ? c - 1 : c;
    T* dst = (c0 == 0 || chain) ? Wc + (int64_t)slot * df : Wp + (int64_t)(slot - kS) * df;
    stage_state<Wide, Wide::Stage, T, A, true>(acc, dst, buf, j0, i0, d, f);
    if (INC && doc) reset(acc);
  }
  template <class A>
  __device__ __forceinline__ void operator()(int ks, A& acc, char* free_stage) const {
    const int done = ks + 1;
    if (done % steps_per_chunk != 0) return;
    const int c = c0 + done / steps_per_chunk;
    if (c >= c1) return;
    boundary(c, acc, free_stage, docs != nullptr && docs[b * k + c] != 0);
  }
};

// An operand whose K steps are taken chunk by chunk in reverse order (the steps
// inside a chunk keep theirs): step ks of the stream reads the operand's step
// (last - t) spc + ks - t spc, t = ks / spc, for chunks of spc steps.
template <class OP>
struct RevChunks : OP {
  int spc, last;
  __device__ __forceinline__ void issue(int ks, char* tile) const {
    const int t = ks / spc;
    OP::issue((last - t) * spc + (ks - t * spc), tile);
  }
};

// NAT: Zt and Vt are Z [B, n, f] and V [B, n, d] in their row-major layout
// (tokens are rows), read as MN-major operands; otherwise the token-contiguous
// copies [B, f, n] and [B, d, n].  REV (with NAT): the chunks are scanned in
// reverse order, last chunk first; state index c then names the c-th chunk of
// that order.
template <typename T, bool NAT, bool REV, bool INC = false>
TTT_GEMM_KERNEL(Wide) void k_chunk_update_scan(const T* __restrict__ Zt, const T* __restrict__ Vt,
                                               const T* __restrict__ W0, T* __restrict__ Wc, T* __restrict__ Wp,
                                               float* __restrict__ Tot, float* __restrict__ Wf, int n, int d, int f,
                                               int C_, int S, const uint8_t* __restrict__ docs,
                                               const float* __restrict__ Winit, int* __restrict__ sync,
                                               int npairs, long long wait) {
  using G = Wide;
  // the operand stages, and one word past them for the chained segments' wait (a second LDS object would
  // cost the K loop its alias information: the fragment reads would then wait for the next step's DMA)
  __shared__ __attribute__((aligned(16))) char smem[G::Smem + 16];
  int* s_ok = reinterpret_cast<int*>(smem + G::Smem);
  const int TP = (f + G::BP - 1) / G::BP, TQ = (d + G::BQ - 1) / G::BQ;
  const int per = TP * TQ;
  const bool chain = sync != nullptr;
  int b, sg, tile, pair = 0;
  if (chain) {
    // S = 2, chained: XCD x (workgroups x, x + 8, ...) takes a contiguous range
    // of the npairs (batch row, state tile) pairs, first their segment-0 tiles,
    // then their segment-1 tiles; the grid is padded to 16 ceil(npairs / 8)
    const int x = (int)(blockIdx.x & 7), L = (int)(blockIdx.x >> 3);
    const int q = npairs >> 3, r = npairs & 7;
    const int np = q + (x < r ? 1 : 0), p0 = x * q + min(x, r);
    if (L >= 2 * np) return;
    sg = L >= np ? 1 : 0;
    pair = p0 + L - sg * np;
    b = pair / per;
    tile = pair - b * per;
  } else {
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int bs = id / per;
    b = bs / S;
    sg = bs - b * S;
    tile = id - bs * per;
  }
  int tp, tq;
  // unchained: every d_model tile of one d_ff tile in one group: the tiles
  // running at the same time then read few distinct Zt rows, and each stretch
  // of the token stream is fetched from HBM about once rather than once per
  // round; chained: chain_group
  grouped_tile(tile, TP, TQ, chain ? chain_group(TQ) : TQ, tp, tq);
  const int k = n / C_, kS = k / S;
  const int c0 = sg * kS;
  const int j0 = tp * G::BP, i0 = tq * G::BQ;
  const int64_t df = (int64_t)d * f;
  const unsigned kbytes = (unsigned)kS * C_ * esz<T>();

  static_assert(NAT || !REV, "the reversed order reads the row-major operands");
  static_assert(!INC || !NAT, "the update-then-apply states: the forward layout");
  using OPP = std::conditional_t<NAT, DmaOpMN<T, G::NW, G::BP>, DmaOp<G::NW, G::BP>>;
  using OPQ = std::conditional_t<NAT, DmaOpMN<T, G::NW, G::BQ>, DmaOp<G::NW, G::BQ>>;
  std::conditional_t<REV, RevChunks<OPP>, OPP> op;
  std::conditional_t<REV, RevChunks<OPQ>, OPQ> oq;
  if constexpr (NAT) {
    // this segment's tokens: chunks c0 .. c0 + kS - 1 of the scan order, stored from chunk pc0 on
    const int pc0 = REV ? k - c0 - kS : c0;
    const int64_t t0 = (int64_t)b * n + (int64_t)pc0 * C_;
    op.init(Zt + t0 * f + j0, min(G::BP, f - j0), (uint64_t)f * esz<T>(), kS * C_);
    oq.init(Vt + t0 * d + i0, min(G::BQ, d - i0), (uint64_t)d * esz<T>(), kS * C_);
    if constexpr (REV) {
      op.spc = oq.spc = C_ * esz<T>() / 128;
      op.last = oq.last = kS - 1;
    }
  } else {
    const uint64_t ldb = (uint64_t)n * esz<T>();
    op.init(Zt + ((int64_t)b * f + j0) * n + (int64_t)c0 * C_, nullptr, min(G::BP, f - j0), ldb, kbytes);
    oq.init(Vt + ((int64_t)b * d + i0) * n + (int64_t)c0 * C_, nullptr, min(G::BQ, d - i0), ldb, kbytes);
  }
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  T* wc = Wc + (int64_t)b * k * df;
  if (sg == 0) {
    // a resumed row (Winit) starts from its own fp32 state unless a document starts at chunk 0
    const float* wi = (Winit != nullptr && !doc_start(docs, b, k, 0, true)) ? Winit + (int64_t)b * df : nullptr;
    for_state_quads<G>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
      const f32x4 w = wi != nullptr ? load4(wi + ro + dj) : load4(W0 + ro + dj);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ib][jb][4 * g + e] = w[e];
    });
    if (!INC) stage_state<G, G::Smem>(acc, wc, smem, j0, i0, d, f);     // chunk 0: W_down0 (or the resumed state)
  } else if (docs != nullptr && docs[(int64_t)b * k + c0] != 0) {
    // a document starts with this segment: its states are absolute from the start (chunk c0's state is
    // written by the fix-up, or, chained, by segment 0)
    for_state_quads<G>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
      const f32x4 w = load4(W0 + ro + dj);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ib][jb][4 * g + e] = w[e];
    });
  }
  const int spc = C_ * esz<T>() / 128, nks = (int)(kbytes / 128);
  const SnapshotHook<T, INC> hook{wc, Wp + (int64_t)b * (k - kS) * df, W0, docs, b, k, spc, c0, c0 + kS, kS, j0,
                                  i0, d, f, chain};
  // Chained segment 1, not starting a document: its first chunk from zero, then the partner's end state is
  // added at the first boundary, outside the K loop (so the loop's registers stay as they are), and its states
  // from there on are absolute.  Every other tile runs the whole loop in the first range.
  const bool split = chain && sg == 1 && !(docs != nullptr && docs[(int64_t)b * k + c0] != 0);
  const SnapshotHook<T, INC> hook1{wc, hook.Wp, W0, docs, b, k, spc, c0, split ? c0 + 1 : c0 + kS, kS, j0, i0, d, f,
                                   chain};
  mainloop_range<T, G>(op, oq, 0, split ? spc : nks, acc, smem, hook1);
  bool failed = false;
  if (split) {
    const bool doc = kS > 1 && docs != nullptr && docs[(int64_t)b * k + c0 + 1] != 0;
    // INC writes chunk c0's state before a reset at c0 + 1, so it always needs the end state
    if (INC || !doc) {
      if (wait_published(sync + pair, wait, s_ok)) {
        const float* tot = Tot + (int64_t)b * df;
        for_state_quads<G>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
          const f32x4 t = load4(tot + ro + dj);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[ib][jb][4 * g + e] += t[e];
        });
      } else {
        failed = true;
      }
    }
    if (kS > 1) hook.boundary(c0 + 1, acc, smem, doc);
  }
  mainloop_range<T, G>(op, oq, split ? spc : nks, nks, acc, smem, hook);
  float* out = sg == S - 1 ? Wf + (int64_t)b * df : Tot + ((int64_t)b * (S - 1) + sg) * df;
  stage_state<G, G::Smem>(acc, out, smem, j0, i0, d, f);
  // INC: the segment's last chunk's state (one or two segments: in Wc)
  if (INC) stage_state<G, G::Smem, T, decltype(acc), true>(acc, wc + (int64_t)(c0 + kS - 1) * df, smem, j0, i0, d, f);
  if (!chain) return;
  if (sg == 0) {
    // chunk kS's state (segment 1's first): this segment's end state, or W_down0 where a document starts there
    // (INC: segment 1 writes every state of its own chunks)
    if (!INC && docs != nullptr && docs[(int64_t)b * k + kS] != 0) {
      for_state_quads<G>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
        const f32x4 w = load4(W0 + ro + dj);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[ib][jb][4 * g + e] = w[e];
      });
    }
    if (!INC) stage_state<G, G::Smem, T, decltype(acc), true>(acc, wc + (int64_t)kS * df, smem, j0, i0, d, f);
    // publish: every wave waits for its stores of the end state (they are then in the XCD's L2), and one
    // release store of the flag (which writes the L2 back for the other XCDs) follows them all
    wait_dma();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(sync + pair, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x == 0) {
    sync[npairs + pair] = failed ? 1 : 0;    // the fix-up completes this tile
  }
}

// Completes a segmented update-scan: adds to every partial state of segments
// 1..S-1, and to W_final, the total of the segments before it, rounding each
// state once to the operand dtype.  With packed documents a state is absolute
// (nothing to add) from the first document start in its segment on, a
// segment's first chunk is W_down0 when a document starts there, and the
// offset carried to the next segment is its absolute end state if a document
// started within it.  Four elements per thread, grid.y = batch.
template <typename T>
__global__ __launch_bounds__(256) void k_scan_fixup(T* __restrict__ Wc, const T* __restrict__ Wp,
                                                    const float* __restrict__ Tot, float* __restrict__ Wf,
                                                    const T* __restrict__ W0, const uint8_t* __restrict__ docs,
                                                    int k, int S, int64_t df) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= df) return;
  const int b = blockIdx.y, kS = k / S;
  T* wc = Wc + (int64_t)b * k * df + e;
  const T* wp = Wp + (int64_t)b * (k - kS) * df + e;
  const float* tot = Tot + (int64_t)b * (S - 1) * df + e;
  f32x4 off = load4(tot);                                   // W_down0 + segment 0 (absolute)
  bool abs_ = false;                                        // a document started in the current segment
  for (int sg = 1; sg < S; ++sg) {
    const int c0 = sg * kS;
    abs_ = doc_start(docs, b, k, c0);
    const f32x4 s0 = abs_ ? load4(W0 + e) : off;
    store4(wc + (int64_t)c0 * df, s0[0], s0[1], s0[2], s0[3]);
    for (int c = c0 + 1; c < c0 + kS; ++c) {
      abs_ = abs_ || doc_start(docs, b, k, c);
      const f32x4 pv = load4(wp + (int64_t)(c - kS) * df);
      if (abs_) store4(wc + (int64_t)c * df, pv[0], pv[1], pv[2], pv[3]);
      else store4(wc + (int64_t)c * df, off[0] + pv[0], off[1] + pv[1], off[2] + pv[2], off[3] + pv[3]);
    }
    if (sg < S - 1) {
      const f32x4 t = load4(tot + (int64_t)sg * df);
      off = abs_ ? t : off + t;
    }
  }
  if (!abs_) {
    float* wf = Wf + (int64_t)b * df + e;
    const f32x4 w = load4(wf);
    store4(wf, w[0] + off[0], w[1] + off[1], w[2] + off[2], w[3] + off[3]);
  }
}

// Completes the tiles of a chained update-scan (S = 2) whose segment 1 did not
// receive its partner's end state in time (status word set): adds segment 0's
// end state Tot to their partial states of chunks kS + 1 .. k - 1 (inc: the
// states after each chunk's step, kS .. k - 1) in place, rounding them a
// second time, and to W_final, up to the first document start in segment 1,
// from where they are absolute.  One workgroup per (batch row,
// state tile) pair; the others return at once.
template <typename T>
__global__ __launch_bounds__(256) void k_chain_fixup(T* __restrict__ Wc, const float* __restrict__ Tot,
                                                     float* __restrict__ Wf, const uint8_t* __restrict__ docs,
                                                     const int* __restrict__ status, int k, int d, int f,
                                                     bool inc) {
  if (status[blockIdx.x] == 0) return;
  const int TP = (f + 255) / 256, TQ = (d + 255) / 256, per = TP * TQ;
  const int b = (int)blockIdx.x / per, tile = (int)blockIdx.x - b * per;
  int tp, tq;
  grouped_tile(tile, TP, TQ, chain_group(TQ), tp, tq);
  const int j0 = tp * 256, i0 = tq * 256, kS = k / 2;
  const int jn = min(256, f - j0), in_ = min(256, d - i0);
  const int64_t df = (int64_t)d * f;
  const float* tot = Tot + (int64_t)b * df;
  int cend = k;                                   // chunks before the first document start after kS are partial
  for (int c = kS + 1; c < k; ++c)
    if (doc_start(docs, b, k, c)) {
      cend = c;
      break;
    }
  const int col = (threadIdx.x & 63) * 4;
  for (int r = threadIdx.x >> 6; r < in_; r += 4) {
    if (col >= jn) continue;                      // jn % 4 == 0
    const int64_t o = (int64_t)(i0 + r) * f + j0 + col;
    const f32x4 t = load4(tot + o);
    for (int c = inc ? kS : kS + 1; c < cend; ++c) {
      T* w = Wc + ((int64_t)b * k + c) * df + o;
      const f32x4 v = load4(w);
      store4(w, v[0] + t[0], v[1] + t[1], v[2] + t[2], v[3] + t[3]);
    }
    if (cend == k) {
      float* w = Wf + (int64_t)b * df + o;
      const f32x4 v = load4(w);
      store4(w, v[0] + t[0], v[1] + t[1], v[2] + t[2], v[3] + t[3]);
    }
  }
}

// ------------------------------------------------------------------ apply

// O_c = Z_c W^T for every chunk (eq. (3)).  P = d_model rows of W, Q = the
// chunk's tokens, K = d_ff.  W of (b, c) is W + b * wsb + c * wsc.  Z is read
// from its token-contiguous copy Zt [B, f, n] (the one the updates contract
// over) as an MN-major operand, so no row-major copy of Z is needed.
// ZNAT: Zt is Z [B, n, f] in its row-major layout, a K-major operand.
template <typename T, bool ZNAT>
TTT_GEMM_KERNEL(Wide) void k_apply(const T* __restrict__ Zt, const T* __restrict__ W, int64_t wsb, int64_t wsc,
                                   T* __restrict__ O, int n, int d, int f, int C_, float oscale) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (d + G::BP - 1) / G::BP, TQ = (C_ + G::BQ - 1) / G::BQ;
  const int per = TP * TQ;
  // chunks of at least 128 tiles: runs of 32 tiles (an XCD's round) in groups of 8 token tiles, 4 x 8 blocks
  // (the whole GPU on about 1.6 chunks at a time); smaller chunks: the plain XCD order
  const bool big = per >= 128;
  const int id = big ? xcd_runs(blockIdx.x, gridDim.x, 32) : xcd_remap(blockIdx.x, gridDim.x);
  const int bc = id / per;
  int tp, tq;
  grouped_tile(id - bc * per, TP, TQ, big ? 8 : 4, tp, tq);
  const int k = n / C_;
  const int b = bc / k, c = bc - b * k;
  const int i0 = tp * G::BP, t0 = tq * G::BQ;
  const int64_t row0 = (int64_t)b * n + (int64_t)c * C_ + t0;
  const uint64_t ldb = (uint64_t)f * esz<T>();

  DmaOp<G::NW, G::BP> op;
  std::conditional_t<ZNAT, DmaOp<G::NW, G::BQ>, DmaOpMN<T, G::NW, G::BQ>> oq;
  op.init(W + (int64_t)b * wsb + (int64_t)c * wsc + (int64_t)i0 * f, nullptr, min(G::BP, d - i0), ldb,
          (unsigned)ldb);
  if constexpr (ZNAT)
    oq.init(Zt + row0 * f, nullptr, min(G::BQ, C_ - t0), ldb, (unsigned)ldb);
  else
    oq.init(Zt + (int64_t)b * f * n + (int64_t)c * C_ + t0, min(G::BQ, C_ - t0), (uint64_t)n * esz<T>(), f);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  // O [token, channel]: staged as [token][channel] (one pass for bf16, two for fp32)
  const int tn = min(G::BQ, C_ - t0), in_ = min(G::BP, d - i0);
  constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(T) + G::Smem - 1) / G::Smem, RPP = G::BQ / PASSES;
  const Staged<T, G::BP> st{smem};
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int j = 0; j < G::NQB; ++j) {
      const int q = G::acc_q(j) - ps * RPP;
      if (q < 0 || q >= RPP) continue;
#pragma unroll
      for (int i = 0; i < G::NPB; ++i)
        st.put4(q, G::acc_p(i, 0), oscale * acc[i][j][0], oscale * acc[i][j][1], oscale * acc[i][j][2],
                oscale * acc[i][j][3]);
    }
    __syncthreads();
    st.template flush<G::NT, RPP, false, 0>(max(0, min(RPP, tn - ps * RPP)), [&](int r, int col) -> T* {
      return col < in_ ? O + (row0 + ps * RPP + r) * d + i0 + col : nullptr;
    });
    __syncthreads();
  }
}

// ------------------------------------------------------------------ backward of the dot chunk loop

// dZ_j = dO_j W_j + eta V^_j S_j for every chunk j, with W_j the state chunk j
// was applied with and S_j = sum_{c>j} dO_c^T Z_c (Method §3's prefix form
// differentiated; see the backward entry point).  P = d_ff columns of the
// [d, f] states (MN-major: f contiguous), Q = the chunk's tokens (rows of
// eta V^ and dO, [n, d]), K = d_model twice: one accumulator takes both
// contractions, a K loop over (S_j, eta V^_j) and then one over (W_j, dO_j),
// each with its own operand state (both live at once spill).  State j sits at
// W + b wsb + j wsc (S likewise; its stride may be negative).  dZ [B, n, f]
// through LDS like O.
// The rows of V and dO are ldq elements apart (d for [n, d] matrices).  QT:
// V and dO are one chunk's token-contiguous [B, d, C] buffers instead (read
// MN-major), and the launch covers chunk cfix of every row only.
template <typename T, bool QT>
TTT_GEMM_KERNEL(Wide) void k_dz(const T* __restrict__ dO, const T* __restrict__ V, const T* __restrict__ W,
                                int64_t wsb, int64_t wsc, const T* __restrict__ S, int64_t ssb, int64_t ssc,
                                T* __restrict__ dZ, int n, int d, int f, int C_, int ldq, int cfix) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (f + G::BP - 1) / G::BP, TQ = (C_ + G::BQ - 1) / G::BQ;
  const int per = TP * TQ;
  const int id = group_sync_tile(blockIdx.x, gridDim.x, per);     // all XCDs on one chunk at a time
  const int bc = id / per;
  int tp, tq;
  grouped_tile(id - bc * per, TP, TQ, 4, tp, tq);
  const int k = QT ? 1 : n / C_;
  const int b = bc / k, c = QT ? cfix : bc - b * k;
  const int j0 = tp * G::BP, t0 = tq * G::BQ;
  const int64_t row0 = (int64_t)b * n + (int64_t)c * C_ + t0;
  const uint64_t ldd = (uint64_t)d * esz<T>(), ldf = (uint64_t)f * esz<T>();
  constexpr int KR = DmaOpMN<T, G::NW, G::BP>::KR;
  const int nks = (d + KR - 1) / KR;
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  // stream 0: (S_j, eta V^_j); stream 1: (W_j, dO_j).  Each K loop ends on a
  // barrier, so the second may refill the stages at once.
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    DmaOpMN<T, G::NW, G::BP> op;
    std::conditional_t<QT, DmaOpMN<T, G::NW, G::BQ>, DmaOp<G::NW, G::BQ>> oq;
    const T* Pm = st == 0 ? S + (int64_t)b * ssb + (int64_t)c * ssc : W + (int64_t)b * wsb + (int64_t)c * wsc;
    const T* Qm = st == 0 ? V : dO;
    op.init(Pm + j0, min(G::BP, f - j0), ldf, d);
    if constexpr (QT) {
      const int64_t q0 = (int64_t)b * d * C_ + t0;               // chunk buffers [B, d, C]
      oq.init(Qm + q0, min(G::BQ, C_ - t0), (uint64_t)C_ * esz<T>(), d);
    } else {
      const uint64_t ldqb = (uint64_t)ldq * esz<T>();
      oq.init(Qm + row0 * ldq, nullptr, min(G::BQ, C_ - t0), ldqb, (unsigned)ldd);
    }
    mainloop<T, G>(op, oq, nks, acc, smem, NoHook{});
  }

  const int tn = min(G::BQ, C_ - t0), jn = min(G::BP, f - j0);
  constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(T) + G::Smem - 1) / G::Smem, RPP = G::BQ / PASSES;
  const Staged<T, G::BP> st{smem};
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
    for (int j = 0; j < G::NQB; ++j) {
      const int q = G::acc_q(j) - ps * RPP;
      if (q < 0 || q >= RPP) continue;
#pragma unroll
      for (int i = 0; i < G::NPB; ++i) st.put4(q, G::acc_p(i, 0), acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
    __syncthreads();
    st.template flush<G::NT, RPP>(max(0, min(RPP, tn - ps * RPP)), [&](int r, int col) -> T* {
      return col < jn ? dZ + (row0 + ps * RPP + r) * f + j0 + col : nullptr;
    });
    __syncthreads();
  }
}

// out [df] = sum over the B rows of Tot (fp32, rows `stride` elements apart),
// four elements per thread.
__global__ __launch_bounds__(256) void k_sum_rows(const float* __restrict__ Tot, float* __restrict__ out, int B,
                                                  int64_t df, int64_t stride) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= df) return;
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) s += load4(Tot + (int64_t)b * stride + e);
  store4(out + e, s[0], s[1], s[2], s[3]);
}

// Document starts of the reversed chunk order, for the suffix scan of the
// backward: reversed chunk t is chunk k - 1 - t, and it starts a document of
// the reversed order when chunk k - t starts one (chunk k - 1 - t ends its
// document); reversed chunk 0 always does.  docs, rd: [B, k].
__global__ __launch_bounds__(256) void k_rev_docs(const uint8_t* __restrict__ docs, uint8_t* __restrict__ rd, int B,
                                                  int k) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)B * k) return;
  const int64_t b = e / k;
  const int t = (int)(e - b * k);
  rd[e] = t == 0 ? 1 : (docs[b * k + (k - t)] != 0 ? 1 : 0);
}

// The state the MSE apply of chunk c reads, kept for a backward pass:
// Ws[b, c] = W_down0 where a document starts (doc_start), else Wcur[b];
// Ws [B, k, d, f], four elements per thread, grid.y = B.
template <typename T>
__global__ __launch_bounds__(256) void k_keep_state(const T* __restrict__ W0, const T* __restrict__ Wcur,
                                                    T* __restrict__ Ws, const uint8_t* __restrict__ docs, bool cont,
                                                    int k, int c, int64_t df) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= df) return;
  const int b = blockIdx.y;
  const T* src = doc_start(docs, b, k, c, cont) ? W0 : Wcur + (int64_t)b * df;
  const f32x4 v = load4(src + e);
  store4(Ws + ((int64_t)b * k + c) * df + e, v[0], v[1], v[2], v[3]);
}

// The MSE backward at a document start (packed rows): where chunk c of row b
// starts a document, the state gradient G[b] = dLoss/dW_c is that document's
// contribution to dW_down0 (dW0 += G[b]) and the previous document's last
// chunk receives none (G[b] = 0, and its operand copy Gsh[b] if any).  A thread
// takes 4 elements of every row, rows in order, so the sum is deterministic.
template <typename T>
__global__ __launch_bounds__(256) void k_doc_grad_reset(float* __restrict__ G, T* __restrict__ Gsh,
                                                        float* __restrict__ dW0, const uint8_t* __restrict__ docs,
                                                        int B, int k, int c, int64_t df, float* __restrict__ dWi) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= df) return;
  f32x4 a = load4(dW0 + e);
  bool any = false;
  for (int b = 0; b < B; ++b) {
    if (dWi != nullptr && c == 0) {     // resumed rows: chunk 0 starts a document only where flagged
      const bool cont = !doc_start(docs, b, k, 0, true);
      const f32x4 g = load4(G + (int64_t)b * df + e);
      store4(dWi + (int64_t)b * df + e, cont ? g[0] : 0.f, cont ? g[1] : 0.f, cont ? g[2] : 0.f, cont ? g[3] : 0.f);
      if (cont) continue;
    }
    if (!doc_start(docs, b, k, c)) continue;
    const int64_t o = (int64_t)b * df + e;
    a += load4(G + o);
    any = true;
    store4(G + o, 0.f, 0.f, 0.f, 0.f);
    if (Gsh != nullptr) store4(Gsh + o, 0.f, 0.f, 0.f, 0.f);
  }
  if (any) store4(dW0 + e, a[0], a[1], a[2], a[3]);
}

// Dot backward of resumed rows: Tt [B, d, f] holds each row's first-document
// gradient (the reversed scan's totals).  A row continues from W_init unless
// chunk 0 is flagged: then dWi[b] = Tt[b] and its first document is no part of
// dW_down0, so it is taken off the all-document sum already in dW0 (have_dW0;
// without packed documents every row continues and dW0 = 0).  Rows flagged at
// chunk 0 get dWi[b] = 0.
__global__ __launch_bounds__(256) void k_resume_split(const float* __restrict__ Tt, const uint8_t* __restrict__ docs,
                                                      float* __restrict__ dW0, float* __restrict__ dWi, int B, int k,
                                                      int64_t df, bool have_dW0) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= df) return;
  f32x4 a = have_dW0 ? load4(dW0 + e) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) {
    const bool cont = !doc_start(docs, b, k, 0, true);
    const f32x4 g = cont ? load4(Tt + (int64_t)b * df + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (have_dW0) a -= g;
    store4(dWi + (int64_t)b * df + e, g[0], g[1], g[2], g[3]);
  }
  store4(dW0 + e, a[0], a[1], a[2], a[3]);
}

// dst = scale * src over n elements, four per thread (n % 4 == 0).  With an
// update mask [B, k] the elements are token rows of `row` elements ([B, n, row],
// chunks of C tokens) and the rows of masked chunks are multiplied by zero.
template <typename T>
__global__ __launch_bounds__(256) void k_scale(const T* __restrict__ src, T* __restrict__ dst, int64_t n,
                                               float scale, const uint8_t* __restrict__ umask, int row, int ntok,
                                               int C_) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  if (umask != nullptr) {
    const int64_t tok = e / row;                    // row % 4 == 0: the four elements share a token
    scale *= update_flag(umask, tok / ntok, ntok / C_, (int)(tok % ntok) / C_);
  }
  const f32x4 v = load4(src + e);
  store4(dst + e, scale * v[0], scale * v[1], scale * v[2], scale * v[3]);
}

// p[0 .. n) = 0, four elements per thread (n % 4 == 0).
template <typename T>
__global__ __launch_bounds__(256) void k_zero(T* __restrict__ p, int64_t n) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e < n) store4(p + e, 0.f, 0.f, 0.f, 0.f);
}

// ------------------------------------------------------------------ MSE objective

// Apply of chunk c with the current state and the residual of its squared error,
// scaled by the step: O_c = Z_c W^T, Rt[b] = rscale (O_c - V^_c)^T [B, d, C]
// with rscale = -eta / C, so that the update is a plain accumulation
// W + Rt Z_c.  P = d_model rows of W (W_down0 where a document starts, else this row's state
// copy), Q = the chunk's tokens, read from Zt [B, f, n] as an MN-major operand,
// K = d_ff.
// GEN (the MSE loop's backward): Rt = rscale O + vscale V^ instead, and O, if
// not null, is written scaled by oscale; O may be null in either form.  ZNAT:
// Zt is Z [B, n, f] as it is (a K-major operand) instead of its
// token-contiguous copy.
template <typename T, bool GEN, bool ZNAT>
TTT_GEMM_KERNEL(Wide) void k_mse_apply(const T* __restrict__ Zt, const T* __restrict__ W0,
                                       const T* __restrict__ Wcur, T* __restrict__ O, const T* __restrict__ Vt,
                                       T* __restrict__ Rt, const uint8_t* __restrict__ docs, int n, int d, int f,
                                       int C_, int c, float rscale, bool cont, const uint8_t* __restrict__ umask,
                                       float vscale, float oscale, int64_t wstride) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (d + G::BP - 1) / G::BP, TQ = (C_ + G::BQ - 1) / G::BQ;
  const int per = TP * TQ;
  const int id = group_sync_tile(blockIdx.x, gridDim.x, per);     // all XCDs on one batch row at a time
  const int b = id / per;
  int tp, tq;
  grouped_tile(id - b * per, TP, TQ, 4, tp, tq);
  const int i0 = tp * G::BP, t0 = tq * G::BQ;
  const int64_t row0 = (int64_t)b * n + (int64_t)c * C_ + t0;
  const uint64_t ldb = (uint64_t)f * esz<T>();
  rscale *= update_flag(umask, b, n / C_, c);       // a masked chunk's update adds zeros
  if constexpr (GEN) oscale *= update_flag(umask, b, n / C_, c);   // (the backward: its target gets no gradient)

  DmaOp<G::NW, G::BP> op;
  std::conditional_t<ZNAT, DmaOp<G::NW, G::BQ>, DmaOpMN<T, G::NW, G::BQ>> oq;
  // the state chunk c is applied with: W_down0 (shared) where a document starts, else this row's state copy
  const T* W = doc_start(docs, b, n / C_, c, cont) ? W0 : Wcur + (int64_t)b * wstride;
  op.init(W + (int64_t)i0 * f, nullptr, min(G::BP, d - i0), ldb, (unsigned)ldb);
  if constexpr (ZNAT)
    oq.init(Zt + row0 * f, nullptr, min(G::BQ, C_ - t0), ldb, (unsigned)ldb);
  else
    oq.init(Zt + (int64_t)b * f * n + (int64_t)c * C_ + t0, min(G::BQ, C_ - t0), (uint64_t)n * esz<T>(), f);
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);
  mainloop<T, G>(op, oq, (int)((ldb + 127) / 128), acc, smem, NoHook{});

  static_assert(G::GPB == 1, "one accumulator group per block");
  const int tn = min(G::BQ, C_ - t0), in_ = min(G::BP, d - i0);

  // O [token, channel]: staged as [token][channel], in passes over token rows
  if (O != nullptr) {
    constexpr int PASSES = (G::BQ * G::BP * (int)sizeof(T) + G::Smem - 1) / G::Smem, RPP = G::BQ / PASSES;
    const Staged<T, G::BP> st{smem};
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
      for (int j = 0; j < G::NQB; ++j) {
        const int q = G::acc_q(j) - ps * RPP;
        if (q < 0 || q >= RPP) continue;
#pragma unroll
        for (int i = 0; i < G::NPB; ++i) {
          const float os = GEN ? oscale : 1.0f;
          st.put4(q, G::acc_p(i, 0), os * acc[i][j][0], os * acc[i][j][1], os * acc[i][j][2], os * acc[i][j][3]);
        }
      }
      __syncthreads();
      st.template flush<G::NT, RPP, false, 0>(max(0, min(RPP, tn - ps * RPP)), [&](int r, int col) -> T* {
        return col < in_ ? O + (row0 + ps * RPP + r) * d + i0 + col : nullptr;
      });
      __syncthreads();
    }
  }
  // Rt [b, channel, token] = rscale (O - V^) in fp32: the accumulators are staged as
  // fp32 [channel][token] rows (in passes over channels); each thread then
  // takes 8 consecutive tokens of one channel, reads V^ from Vt in one or two
  // 16-byte pieces, subtracts and writes the same span of Rt.  Skipped when
  // Rt is null (an apply with no residual).
  if (Rt != nullptr) {
    constexpr int RPP = G::Smem / (G::BQ * 4);        // channel rows per pass
    constexpr int PASSES = G::BP / RPP;
    constexpr int SPANS = G::BQ / 8;                  // 8-token spans per row
    const Staged<float, G::BQ> st{smem};
    const T* vt = Vt + ((int64_t)b * d + i0) * n + (int64_t)c * C_ + t0;
    T* rt = Rt + ((int64_t)b * d + i0) * C_ + t0;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
      for (int i = 0; i < G::NPB; ++i) {
        const int p = G::acc_p(i, 0) - ps * RPP;
        if (p < 0 || p >= RPP) continue;
#pragma unroll
        for (int j = 0; j < G::NQB; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) st.put1(p + e, G::acc_q(j), acc[i][j][e]);
      }
      __syncthreads();
      const int rows = max(0, min(RPP, in_ - ps * RPP));
      // KB spans per thread and trip, their V^ loads all issued before any
      // is used (one memory latency per trip rather than per span)
      constexpr int KB = 4;
      for (int i0s = threadIdx.x; i0s < rows * SPANS; i0s += KB * G::NT) {
        f32x4 v0[KB], v1[KB];
        int rr[KB], tt[KB];
        bool ok[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const int idx = i0s + k * G::NT;
          rr[k] = idx / SPANS;
          tt[k] = (idx - rr[k] * SPANS) * 8;
          ok[k] = idx < rows * SPANS && tt[k] < tn;     // tn % 8 == 0
          if (ok[k]) {
            const T* vp = vt + (int64_t)(ps * RPP + rr[k]) * n + tt[k];
            v0[k] = load4(vp);
            v1[k] = load4(vp + 4);
          }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          if (!ok[k]) continue;
          const int r = rr[k], t = tt[k];
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(smem + st.off(r, t));
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(smem + st.off(r, t + 4));
          T* dst = rt + (int64_t)(ps * RPP + r) * C_ + t;
          if constexpr (GEN) {
            store4(dst, rscale * o0[0] + vscale * v0[k][0], rscale * o0[1] + vscale * v0[k][1],
                   rscale * o0[2] + vscale * v0[k][2], rscale * o0[3] + vscale * v0[k][3]);
            store4(dst + 4, rscale * o1[0] + vscale * v1[k][0], rscale * o1[1] + vscale * v1[k][1],
                   rscale * o1[2] + vscale * v1[k][2], rscale * o1[3] + vscale * v1[k][3]);
          } else {
            store4(dst, rscale * (o0[0] - v0[k][0]), rscale * (o0[1] - v0[k][1]), rscale * (o0[2] - v0[k][2]),
                   rscale * (o0[3] - v0[k][3]));
            store4(dst + 4, rscale * (o1[0] - v1[k][0]), rscale * (o1[1] - v1[k][1]), rscale * (o1[2] - v1[k][2]),
                   rscale * (o1[3] - v1[k][3]));
          }
        }
      }
      __syncthreads();
    }
  }
}

// W_{c+1} = W_c - (eta / C) R_c^T Z_c (eq. (4) with the squared error at the
// pre-update state), as W_c + Rt Z_c with Rt already scaled by -eta / C.
// P = d_ff rows of Zt (the chunk's tokens), Q = d_model rows of Rt, K = C.
// The accumulator starts at the state -- W_down0 where a document starts, else the fp32
// state Ws [B, d, f] -- read before the K loop, while its first operands are
// in flight; the result goes out through LDS as whole rows: the fp32 state,
// and into Wsh (may be null) a dtype copy for the next apply.  The fp32 state
// is read and written with non-temporal accesses: it is next used by the
// following chunk's update, and at long-context sizes it is larger than the
// caches, which are better kept for the operands and for Wsh (read next).
// ZNAT: Zt is Z [B, n, f] as it is (an MN-major operand: d_ff contiguous, the
// chunk's tokens as the K rows) instead of its token-contiguous copy.
template <typename T, bool ZNAT>
TTT_GEMM_KERNEL(Wide) void k_mse_update(const T* __restrict__ Zt, const T* __restrict__ Rt, const T* __restrict__ W0,
                                        float* __restrict__ Ws, T* __restrict__ Wsh, const uint8_t* __restrict__ docs,
                                        int n, int d, int f, int C_, int c, bool cont) {
  using G = Wide;
  __shared__ __attribute__((aligned(16))) char smem[G::Smem];
  const int TP = (f + G::BP - 1) / G::BP, TQ = (d + G::BQ - 1) / G::BQ;
  const int per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per;
  int tp, tq;
  grouped_tile(id - b * per, TP, TQ, 4, tp, tq);
  const int j0 = tp * G::BP, i0 = tq * G::BQ;
  const unsigned kbytes = (unsigned)C_ * esz<T>();

  std::conditional_t<ZNAT, DmaOpMN<T, G::NW, G::BP>, DmaOp<G::NW, G::BP>> op;
  DmaOp<G::NW, G::BQ> oq;
  if constexpr (ZNAT)
    op.init(Zt + ((int64_t)b * n + (int64_t)c * C_) * f + j0, min(G::BP, f - j0), (uint64_t)f * esz<T>(), C_);
  else
    op.init(Zt + ((int64_t)b * f + j0) * n + (int64_t)c * C_, nullptr, min(G::BP, f - j0), (uint64_t)n * esz<T>(),
            kbytes);
  oq.init(Rt + ((int64_t)b * d + i0) * C_, nullptr, min(G::BQ, d - i0), (uint64_t)kbytes, kbytes);
  float* ws = Ws + (int64_t)b * d * f;
  typename G::Frag acc[G::NPB][G::NQB];
  zero_acc<G>(acc);                       // entries outside the state stay zero (never stored)
  const bool fresh = doc_start(docs, b, n / C_, c, cont);
  for_state_quads<G>(j0, i0, d, f, [&](int64_t ro, int dj, int ib, int jb, int g) {
    const f32x4 w = fresh ? load4(W0 + ro + dj) : load4_stream(ws + ro + dj);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[ib][jb][4 * g + e] = w[e];
  });
  mainloop<T, G>(op, oq, (int)((kbytes + 127) / 128), acc, smem, NoHook{});

  stage_state<G, G::Smem, float, decltype(acc), true, 8>(acc, ws, smem, j0, i0, d, f);
  if (Wsh != nullptr)
    stage_state<G, G::Smem, T, decltype(acc), false, 8>(acc, Wsh + (int64_t)b * d * f, smem, j0, i0, d, f);
}

// ------------------------------------------------------------------ launchers

static inline unsigned tiles_u(int64_t t) { return (unsigned)t; }
constexpr int kWB = Wide::BP;       // 256 x 256 tiles
static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename T>
hipError_t launch_conv(const T* X0, const T* cw, T* Y, int64_t rows, int n, int d, int K, const uint8_t* docs, int C,
                       bool fwd, const T* halo, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int64_t threads = (rows / kConvRows) * (d / Vec<T>::V);     // rows % kConvRows == 0 (n % 8 == 0)
  const dim3 g((unsigned)cdiv(threads, 256));
  switch (K) {
#define TTT_KW(KW)                                                                                            \
  case KW:                                                                                                    \
    if (fwd) k_conv<T, KW, true><<<g, 256, 0, s>>>(X0, cw, Y, rows, n, d, docs, C, halo);                   \
    else k_conv<T, KW, false><<<g, 256, 0, s>>>(X0, cw, Y, rows, n, d, docs, C, halo);                      \
    break;
    TTT_KW(1) TTT_KW(2) TTT_KW(3) TTT_KW(4) TTT_KW(5) TTT_KW(6) TTT_KW(7) TTT_KW(8)
#undef TTT_KW
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_bwd(const T* X0, const T* cw, const T* dY, T* dX0, float* part, int64_t rows, int n, int d,
                           int K, hipStream_t s, const uint8_t* docs, int C, bool fwd, const T* halo, T* dhalo) {
  if (rows == 0) return hipSuccess;
  const int64_t threads = conv_bwd_partials(rows) * (d / Vec<T>::V);
  const dim3 g((unsigned)cdiv(threads, 256));
  switch (K) {
#define TTT_KW(KW)                                                                                            \
  case KW:                                                                                                    \
    if (fwd)                                                                                                  \
      k_conv_bwd<T, KW, true><<<g, 256, 0, s>>>(X0, cw, dY, dX0, part, rows, n, d, docs, C, nullptr, dhalo);  \
    else                                                                                                      \
      k_conv_bwd<T, KW, false><<<g, 256, 0, s>>>(X0, cw, dY, dX0, part, rows, n, d, docs, C, halo, dhalo);    \
    break;
    TTT_KW(1) TTT_KW(2) TTT_KW(3) TTT_KW(4) TTT_KW(5) TTT_KW(6) TTT_KW(7) TTT_KW(8)
#undef TTT_KW
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_produce_z_bwd(const T* H, const T* Wg, const T* Wu, const T* dZ, T* G, int64_t rows, int n, int d,
                                int f, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  k_produce_z_bwd<T><<<tiles_u(cdiv(rows, kWB) * cdiv(f, kWB / 2)), Wide::NT, 0, s>>>(H, Wg, Wu, dZ, G, rows, n, d,
                                                                                      f);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_transpose(const T* src, T* dst, int batch, int R, int Cs, float scale, int rev, hipStream_t s,
                            const uint8_t* umask, int chunk) {
  if (batch == 0 || R == 0 || Cs == 0) return hipSuccess;
  k_transpose<T><<<dim3((unsigned)(cdiv(Cs, 64) * cdiv(R, 64)), (unsigned)batch), 256, 0, s>>>(
      src, dst, R, Cs, scale, rev, chunk > 0 ? umask : nullptr, chunk);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_produce_z(const T* H, const T* Wg, const T* Wu, T* Z, T* Zt, int64_t rows, int n, int d, int f,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  k_produce_z<T><<<tiles_u(cdiv(rows, kWB) * cdiv(f, kWB / 2)), Wide::NT, 0, s>>>(H, Wg, Wu, Z, Zt, rows, n, d, f);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_produce_vhat(const T* Y, const T* WtT, T* Vt, int64_t rows, int n, int d, float scale,
                               hipStream_t s, const uint8_t* umask, int C) {
  if (rows == 0) return hipSuccess;
  k_produce_vhat<T><<<tiles_u(cdiv(rows, kWB) * cdiv(d, kWB)), Wide::NT, 0, s>>>(Y, WtT, Vt, rows, n, d, scale,
                                                                                  C > 0 ? umask : nullptr, C);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_chunk_delta(const T* Zt, const T* Vt, float* dW, int B, int n, int d, int f, int Cs, hipStream_t s) {
  const int64_t tiles = cdiv(f, kWB) * cdiv(d, kWB) * B * (n / Cs);
  if (tiles == 0) return hipSuccess;
  k_chunk_delta<T><<<tiles_u(tiles), Wide::NT, 0, s>>>(Zt, Vt, dW, n, d, f, Cs);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_chunk_scan(const float* dW, const T* W0, T* Wc, float* Wf, int B, int k, int64_t df, float eta,
                             const uint8_t* docs, const float* Winit, hipStream_t s, bool inclusive) {
  if (B == 0) return hipSuccess;
  k_chunk_scan<T><<<dim3((unsigned)cdiv(df / 4, 256), (unsigned)B), 256, 0, s>>>(dW, W0, Wc, Wf, k, df, eta, docs,
                                                                                 Winit, inclusive);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_flags(int* __restrict__ p, int n) {
  const int i = (int)(blockIdx.x * 256 + threadIdx.x);
  if (i < n) p[i] = 0;
}

// Wall-clock ticks a chained segment waits for its partner: 20 ms, or
// TTT_UPDATE_SCAN_WAIT_US microseconds from the environment (negative: never
// wait, so every tile takes the fix-up path -- for tests of that path).
static long long chain_wait_ticks() {
  long long us = 20000;
  if (const char* v = std::getenv("TTT_UPDATE_SCAN_WAIT_US")) us = std::atoll(v);
  if (us < 0) return -1;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) !=
      hipSuccess || khz <= 0)
    khz = 100000;
  return us * khz / 1000;
}

template <typename T>
hipError_t launch_chunk_update_scan(const T* Zt, const T* Vt, const T* W0, T* Wc, float* Wf, T* Wp, float* Tot,
                                    int B, int n, int d, int f, int Cs, int S, const uint8_t* docs,
                                    const float* Winit, hipStream_t s, int layout, bool inclusive) {
  const int64_t per = cdiv(f, kWB) * cdiv(d, kWB);
  const int64_t tiles = per * B * S;
  if (tiles == 0) return hipSuccess;
  if (inclusive && (S > 2 || layout != kScanTokenContiguous)) return hipErrorInvalidValue;
  // Two segments are chained (no partial states) when the partial-state space
  // holds the flags and status words: 2 npairs ints.
  const int k = n / Cs;
  const int64_t npairs = per * B;
  const bool chain = S == 2 && (int64_t)B * (k - k / 2) * d * f * (int64_t)sizeof(T) >= 8 * npairs;
  if (inclusive && S == 2 && !chain) return hipErrorInvalidValue;
  int* sync = chain ? reinterpret_cast<int*>(Wp) : nullptr;
  const long long wait = chain ? chain_wait_ticks() : 0;
  const unsigned grid = chain ? tiles_u(16 * cdiv(npairs, 8)) : tiles_u(tiles);
  if (chain) {
    k_zero_flags<<<(unsigned)cdiv(npairs, 256), 256, 0, s>>>(sync, (int)npairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define TTT_SCAN_ARGS Zt, Vt, W0, Wc, Wp, Tot, Wf, n, d, f, Cs, S, docs, Winit, sync, (int)npairs, wait
  if (layout == kScanRowMajorReversed)
    k_chunk_update_scan<T, true, true><<<grid, Wide::NT, 0, s>>>(TTT_SCAN_ARGS);
  else if (layout == kScanRowMajor)
    k_chunk_update_scan<T, true, false><<<grid, Wide::NT, 0, s>>>(TTT_SCAN_ARGS);
  else if (inclusive)
    k_chunk_update_scan<T, false, false, true><<<grid, Wide::NT, 0, s>>>(TTT_SCAN_ARGS);
  else
    k_chunk_update_scan<T, false, false><<<grid, Wide::NT, 0, s>>>(TTT_SCAN_ARGS);
#undef TTT_SCAN_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  if (chain) {
    k_chain_fixup<T><<<(unsigned)npairs, 256, 0, s>>>(Wc, Tot, Wf, docs, sync + npairs, k, d, f, inclusive);
    return hipGetLastError();
  }
  const int64_t df = (int64_t)d * f;
  k_scan_fixup<T><<<dim3((unsigned)cdiv(df / 4, 256), (unsigned)B), 256, 0, s>>>(Wc, Wp, Tot, Wf, W0, docs, k, S,
                                                                                  df);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_apply(const T* Zt, const T* W, int64_t wsb, int64_t wsc, T* O, int B, int n, int d, int f, int Cs,
                        float oscale, hipStream_t s, bool znat) {
  const int64_t tiles = cdiv(d, kWB) * cdiv(Cs, kWB) * B * (n / Cs);
  if (tiles == 0) return hipSuccess;
  if (znat)
    k_apply<T, true><<<tiles_u(tiles), Wide::NT, 0, s>>>(Zt, W, wsb, wsc, O, n, d, f, Cs, oscale);
  else
    k_apply<T, false><<<tiles_u(tiles), Wide::NT, 0, s>>>(Zt, W, wsb, wsc, O, n, d, f, Cs, oscale);
  return hipGetLastError();
}

hipError_t launch_rev_docs(const uint8_t* docs, uint8_t* rd, int B, int k, hipStream_t s) {
  if ((int64_t)B * k == 0) return hipSuccess;
  k_rev_docs<<<(unsigned)cdiv((int64_t)B * k, 256), 256, 0, s>>>(docs, rd, B, k);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_scale(const T* src, T* dst, int64_t n, float scale, hipStream_t s, const uint8_t* umask, int row,
                        int ntok, int C) {
  if (n == 0) return hipSuccess;
  k_scale<T><<<(unsigned)cdiv(n / 4, 256), 256, 0, s>>>(src, dst, n, scale, umask, row, ntok, C);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dz(const T* dO, const T* V, const T* W, int64_t wsb, int64_t wsc, const T* S, int64_t ssb,
                     int64_t ssc, T* dZ, int B, int n, int d, int f, int Cs, hipStream_t s, int ldq) {
  const int64_t tiles = cdiv(f, kWB) * cdiv(Cs, kWB) * B * (n / Cs);
  if (tiles == 0) return hipSuccess;
  k_dz<T, false><<<tiles_u(tiles), Wide::NT, 0, s>>>(dO, V, W, wsb, wsc, S, ssb, ssc, dZ, n, d, f, Cs,
                                                      ldq > 0 ? ldq : d, 0);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dz_chunk(const T* Tt, const T* Rt, const T* W, int64_t wsb, const T* S, int64_t ssb, T* dZ, int B,
                           int n, int d, int f, int Cs, int c, hipStream_t s) {
  const int64_t tiles = cdiv(f, kWB) * cdiv(Cs, kWB) * B;
  if (tiles == 0) return hipSuccess;
  k_dz<T, true><<<tiles_u(tiles), Wide::NT, 0, s>>>(Tt, Rt, W, wsb, 0, S, ssb, 0, dZ, n, d, f, Cs, d, c);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mse_apply_gen(const T* Zt, const T* Vt, const T* W0, const T* Wcur, T* O, T* Rt, bool cont, int B,
                                int n, int d, int f, int Cs, int c, float rscale, float vscale, float oscale, bool gen,
                                hipStream_t s, int64_t wstride, const uint8_t* umask) {
  const unsigned g = tiles_u(cdiv(Cs, kWB) * cdiv(d, kWB) * B);
  const int64_t df = (int64_t)d * f;
  if (gen)
    k_mse_apply<T, true, true><<<g, Wide::NT, 0, s>>>(Zt, W0, Wcur, O, Vt, Rt, nullptr, n, d, f, Cs, c, rscale,
                                                      cont, umask, vscale, oscale, wstride > 0 ? wstride : df);
  else
    k_mse_apply<T, false, true><<<g, Wide::NT, 0, s>>>(Zt, W0, Wcur, O, Vt, Rt, nullptr, n, d, f, Cs, c, rscale,
                                                       cont, umask, 0.f, 1.f, wstride > 0 ? wstride : df);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_keep_state(const T* W0, const T* Wcur, T* Ws, const uint8_t* docs, bool cont, int B, int k, int c,
                             int64_t df, hipStream_t s) {
  if (B == 0 || df == 0) return hipSuccess;
  k_keep_state<T><<<dim3((unsigned)cdiv(df / 4, 256), (unsigned)B), 256, 0, s>>>(W0, Wcur, Ws, docs, cont, k, c, df);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_doc_grad_reset(float* G, T* Gsh, float* dW0, const uint8_t* docs, int B, int k, int c, int64_t df,
                                 hipStream_t s, float* dWi) {
  if (B == 0 || df == 0) return hipSuccess;
  k_doc_grad_reset<T><<<(unsigned)cdiv(df / 4, 256), 256, 0, s>>>(G, Gsh, dW0, docs, B, k, c, df, dWi);
  return hipGetLastError();
}

hipError_t launch_resume_split(const float* Tt, const uint8_t* docs, float* dW0, float* dWi, int B, int k, int64_t df,
                               bool have_dW0, hipStream_t s) {
  if (B == 0 || df == 0) return hipSuccess;
  k_resume_split<<<(unsigned)cdiv(df / 4, 256), 256, 0, s>>>(Tt, docs, dW0, dWi, B, k, df, have_dW0);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mse_update(const T* Zt, const T* Rt, const T* W0, float* Ws, T* Wsh, bool cont, int B, int n, int d,
                             int f, int Cs, int c, hipStream_t s) {
  k_mse_update<T, true><<<tiles_u(cdiv(f, kWB) * cdiv(d, kWB) * B), Wide::NT, 0, s>>>(Zt, Rt, W0, Ws, Wsh, nullptr, n,
                                                                                     d, f, Cs, c, cont);
  return hipGetLastError();
}

hipError_t launch_sum_rows(const float* Tot, float* out, int B, int64_t df, hipStream_t s, int64_t stride) {
  if (df == 0) return hipSuccess;
  k_sum_rows<<<(unsigned)cdiv(df / 4, 256), 256, 0, s>>>(Tot, out, B, df, stride > 0 ? stride : df);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_zero(T* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  k_zero<T><<<(unsigned)cdiv(n / 4, 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mse_chunk(const T* Zt, const T* Vt, const T* W0, const T* Wcur, float* Ws, T* Wsh, T* O,
                            T* Rt, const uint8_t* docs, bool cont, int B, int n, int d, int f, int Cs, int c,
                            float eta, hipStream_t s, const uint8_t* umask, bool znat) {
  const unsigned ga = tiles_u(cdiv(Cs, kWB) * cdiv(d, kWB) * B), gu = tiles_u(cdiv(f, kWB) * cdiv(d, kWB) * B);
  if (znat)
    k_mse_apply<T, false, true><<<ga, Wide::NT, 0, s>>>(Zt, W0, Wcur, O, Vt, Rt, docs, n, d, f, Cs, c,
                                                        -eta / (float)Cs, cont, umask, 0.f, 1.f, (int64_t)d * f);
  else
    k_mse_apply<T, false, false><<<ga, Wide::NT, 0, s>>>(Zt, W0, Wcur, O, Vt, Rt, docs, n, d, f, Cs, c,
                                                         -eta / (float)Cs, cont, umask, 0.f, 1.f, (int64_t)d * f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (znat)
    k_mse_update<T, true><<<gu, Wide::NT, 0, s>>>(Zt, Rt, W0, Ws, Wsh, docs, n, d, f, Cs, c, cont);
  else
    k_mse_update<T, false><<<gu, Wide::NT, 0, s>>>(Zt, Rt, W0, Ws, Wsh, docs, n, d, f, Cs, c, cont);
  return hipGetLastError();
}

// The update-then-apply order's apply: O_c = Z_c W^T with the state chunk c's
// step left (Wcur, this row's copy), no residual.
template <typename T>
hipError_t launch_mse_apply_state(const T* Zt, const T* Wcur, T* O, int B, int n, int d, int f, int Cs, int c,
                                  hipStream_t s) {
  const unsigned ga = tiles_u(cdiv(Cs, kWB) * cdiv(d, kWB) * B);
  k_mse_apply<T, false, false><<<ga, Wide::NT, 0, s>>>(Zt, Wcur, Wcur, O, nullptr, nullptr, nullptr, n, d, f, Cs, c,
                                                       0.f, true, nullptr, 0.f, 1.f, (int64_t)d * f);
  return hipGetLastError();
}

// The states a resumed MSE scan starts from: Wf[b] = Winit[b] (fp32) and, for
// a dtype operand, Wsh[b] its rounded copy for the first apply.
template <typename T>
__global__ __launch_bounds__(256) void k_state_copy(const float* __restrict__ Winit, float* __restrict__ Wf,
                                                    T* __restrict__ Wsh, int64_t df) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= df) return;
  const int64_t o = (int64_t)blockIdx.y * df + e;
  const f32x4 w = load4(Winit + o);
  store4(Wf + o, w[0], w[1], w[2], w[3]);
  if (Wsh != nullptr) store4(Wsh + o, w[0], w[1], w[2], w[3]);
}

template <typename T>
hipError_t launch_state_copy(const float* Winit, float* Wf, T* Wsh, int B, int64_t df, hipStream_t s) {
  if (B == 0 || df == 0) return hipSuccess;
  k_state_copy<T><<<dim3((unsigned)cdiv(df / 4, 256), (unsigned)B), 256, 0, s>>>(Winit, Wf, Wsh, df);
  return hipGetLastError();
}

#define TTT_INST(T)                                                                                               \
  template hipError_t launch_conv<T>(const T*, const T*, T*, int64_t, int, int, int, const uint8_t*, int, bool,  \
                                     const T*, hipStream_t);                                                      \
  template hipError_t launch_transpose<T>(const T*, T*, int, int, int, float, int, hipStream_t, const uint8_t*,   \
                                          int);                                                                   \
  template hipError_t launch_produce_z<T>(const T*, const T*, const T*, T*, T*, int64_t, int, int, int,          \
                                          hipStream_t);                                                           \
  template hipError_t launch_produce_vhat<T>(const T*, const T*, T*, int64_t, int, int, float, hipStream_t,      \
                                             const uint8_t*, int);                                                \
  template hipError_t launch_chunk_delta<T>(const T*, const T*, float*, int, int, int, int, int, hipStream_t);   \
  template hipError_t launch_chunk_scan<T>(const float*, const T*, T*, float*, int, int, int64_t, float,         \
                                           const uint8_t*, const float*, hipStream_t, bool);                      \
  template hipError_t launch_chunk_update_scan<T>(const T*, const T*, const T*, T*, float*, T*, float*, int,      \
                                                  int, int, int, int, int, const uint8_t*, const float*,          \
                                                  hipStream_t, int, bool);                                        \
  template hipError_t launch_apply<T>(const T*, const T*, int64_t, int64_t, T*, int, int, int, int, int, float,   \
                                      hipStream_t, bool);                                                         \
  template hipError_t launch_scale<T>(const T*, T*, int64_t, float, hipStream_t, const uint8_t*, int, int, int);  \
  template hipError_t launch_dz<T>(const T*, const T*, const T*, int64_t, int64_t, const T*, int64_t, int64_t, T*, \
                                   int, int, int, int, int, hipStream_t, int);                                    \
  template hipError_t launch_dz_chunk<T>(const T*, const T*, const T*, int64_t, const T*, int64_t, T*, int, int,  \
                                         int, int, int, int, hipStream_t);                                        \
  template hipError_t launch_mse_apply_gen<T>(const T*, const T*, const T*, const T*, T*, T*, bool, int, int, int, \
                                              int, int, int, float, float, float, bool, hipStream_t, int64_t,     \
                                              const uint8_t*);                                                    \
  template hipError_t launch_doc_grad_reset<T>(float*, T*, float*, const uint8_t*, int, int, int, int64_t,       \
                                               hipStream_t, float*);                                              \
  template hipError_t launch_keep_state<T>(const T*, const T*, T*, const uint8_t*, bool, int, int, int, int64_t,  \
                                           hipStream_t);                                                          \
  template hipError_t launch_mse_update<T>(const T*, const T*, const T*, float*, T*, bool, int, int, int, int, int, \
                                           int, hipStream_t);                                                     \
  template hipError_t launch_produce_z_bwd<T>(const T*, const T*, const T*, const T*, T*, int64_t, int, int, int,  \
                                              hipStream_t);                                                       \
  template hipError_t launch_conv_bwd<T>(const T*, const T*, const T*, T*, float*, int64_t, int, int, int,        \
                                         hipStream_t, const uint8_t*, int, bool, const T*, T*);                   \
  template hipError_t launch_zero<T>(T*, int64_t, hipStream_t);                                                   \
  template hipError_t launch_mse_apply_state<T>(const T*, const T*, T*, int, int, int, int, int, int,          \
                                                hipStream_t);                                                     \
  template hipError_t launch_mse_chunk<T>(const T*, const T*, const T*, const T*, float*, T*, T*, T*,             \
                                          const uint8_t*, bool, int, int, int, int, int, int, float, hipStream_t,  \
                                          const uint8_t*, bool);                                                  \
  template hipError_t launch_state_copy<T>(const float*, float*, T*, int, int64_t, hipStream_t);
TTT_INST(float)
TTT_INST(bf16)
#undef TTT_INST

}  // namespace ttt
