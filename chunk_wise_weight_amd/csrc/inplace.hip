// In-Place TTT kernels for gfx950: the producers of Z and V^, the dot-objective
// deltas / prefix scan / fused update-scan, the apply, and the MSE chunk scan.
// Layer semantics: review of "In-Place Test-Time Training", Method §1-§3.
#include "gemm.hpp"
#include "launch.hpp"

namespace ttt {

// ------------------------------------------------------------------ producers

// Z = silu(H W_gate^T) * (H W_up^T)  (eq. (2)).
// P = rows of W_gate / W_up interleaved in 32-row blocks (gate, up, gate, up,
// ...): a 256-row P tile covers 128 output columns, and each lane holds the
// gate and the up value of the same output in blocks i and i + 1.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_produce_z(const T* __restrict__ H, const T* __restrict__ Wg,
                                                         const T* __restrict__ Wu, T* __restrict__ Z,
                                                         int64_t rows, int d, int f) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int TP = (f + 127) / 128;
  const int TQ = (int)((rows + kTile - 1) / kTile);
  int tp, tq;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), TP, TQ, 4, tp, tq);

  LoadKC<T> lp, lq;
  lp.init([&](int r) -> const T* {
    int blk = r >> 5;
    int j = tp * 128 + (blk >> 1) * 32 + (r & 31);
    if (j >= f) return nullptr;
    return ((blk & 1) ? Wu : Wg) + (int64_t)j * d;
  }, d);
  lq.init([&](int r) -> const T* {
    int64_t t = (int64_t)tq * kTile + r;
    return t < rows ? H + t * d : nullptr;
  }, d);
  f32x16 acc[4][4];
  mainloop<T>(lp, lq, (d + LoadKC<T>::BK - 1) / LoadKC<T>::BK, acc, smem, NoHook{});

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int ii = 0; ii < 4; ii += 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = (int64_t)tq * kTile + acc_q(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = tp * 128 + ((w >> 1) * 2 + (ii >> 1)) * 32 + g * 8 + (lane >> 5) * 4;
        if (row < rows && col < f) {
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] = silu_f(acc[ii][j][4 * g + e]) * acc[ii + 1][j][4 * g + e];
          store4(Z + row * f + col, z[0], z[1], z[2], z[3]);
        }
      }
    }
  }
}

// Q-operand loader that forms Y = CausalDepthwiseConv1D_KW(X0) on the fly:
// chunk (row t, channels ch..ch+V) = sum_j conv_w[ch.., j] * X0[t-(KW-1)+j, ch..],
// rows before the start of the sequence are zero.
template <typename T, int KW>
struct LoadConv {
  static constexpr int V = Vec<T>::V;
  static constexpr int BK = 8 * V;
  static constexpr int N = kTile * 8 / kThreads;
  u32x4 r[N];
  const T* rowp[N];
  int pos[N];
  const T* convw;
  int kc, d;

  __device__ __forceinline__ void init(const T* X0, const T* cw, int64_t rows, int n, int d_, int64_t row0) {
    kc = threadIdx.x & 7;
    d = d_;
    convw = cw;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int64_t t = row0 + i * 32 + (threadIdx.x >> 3);
      rowp[i] = t < rows ? X0 + t * d : nullptr;
      pos[i] = (int)(t % n);
    }
  }
  __device__ __forceinline__ void load(int ks) {
    const int ch = ks * BK + kc * V;
    if (ch >= d) {
#pragma unroll
      for (int i = 0; i < N; ++i) r[i] = (u32x4){0u, 0u, 0u, 0u};
      return;
    }
    // taps of channels ch..ch+V-1: V * KW contiguous elements of conv_w [d, KW]
    float w[V][KW];
    {
      constexpr int NCH = V * KW / Vec<T>::V;   // 16-byte chunks
      const u32x4* src = reinterpret_cast<const u32x4*>(convw + (int64_t)ch * KW);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        u32x4 x = src[c];
        float f[Vec<T>::V];
        if constexpr (sizeof(T) == 2) unpack8(x, f);
        else {
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
        }
#pragma unroll
        for (int e = 0; e < Vec<T>::V; ++e) {
          const int idx = c * Vec<T>::V + e;
          w[idx / KW][idx % KW] = f[e];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float y[V];
#pragma unroll
      for (int v = 0; v < V; ++v) y[v] = 0.f;
      if (rowp[i] != nullptr) {
#pragma unroll
        for (int j = 0; j < KW; ++j) {
          const int back = KW - 1 - j;
          if (pos[i] >= back) {
            u32x4 x = *reinterpret_cast<const u32x4*>(rowp[i] - (int64_t)back * d + ch);
            float xf[V];
            if constexpr (sizeof(T) == 2) unpack8(x, xf);
            else {
#pragma unroll
              for (int e = 0; e < 4; ++e) xf[e] = __uint_as_float(x[e]);
            }
#pragma unroll
            for (int v = 0; v < V; ++v) y[v] = fmaf(w[v][j], xf[v], y[v]);
          }
        }
      }
      u32x4 o;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = bf16_bits_rne(y[2 * e]) | (bf16_bits_rne(y[2 * e + 1]) << 16);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(y[e]);
      }
      r[i] = o;
    }
  }
  __device__ __forceinline__ void store(char* tile) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      *reinterpret_cast<u32x4*>(tile + lds_off(i * 32 + (threadIdx.x >> 3), kc)) = r[i];
  }
};

// V^ = Conv1D(X0) W_target  (eq. (5)); W_target [d_in, d_out] is read
// MN-contiguously as the P operand (rows = output channels).
template <typename T, int KW>
__global__ __launch_bounds__(kThreads) void k_produce_vhat(const T* __restrict__ X0, const T* __restrict__ convw,
                                                            const T* __restrict__ Wt, T* __restrict__ Vh,
                                                            int64_t rows, int n, int d) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int TP = (d + kTile - 1) / kTile;
  const int TQ = (int)((rows + kTile - 1) / kTile);
  int tp, tq;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), TP, TQ, 4, tp, tq);

  LoadMC<T> lp;
  lp.init(Wt + tp * kTile, d, d - tp * kTile, d);
  LoadConv<T, KW> lq;
  lq.init(X0, convw, rows, n, d, (int64_t)tq * kTile);
  f32x16 acc[4][4];
  mainloop<T>(lp, lq, (d + LoadKC<T>::BK - 1) / LoadKC<T>::BK, acc, smem, NoHook{});

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = (int64_t)tq * kTile + acc_q(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = tp * kTile + acc_p(i, g);
        if (row < rows && col < d)
          store4(Vh + row * d + col, acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      }
    }
}

// ------------------------------------------------------------------ dot objective: deltas, scan

// Writes base[q][p] = w0[q][p] + eta * acc for this lane's values (ld = f).
template <typename T, typename TO>
__device__ __forceinline__ void write_state(const f32x16 (&acc)[4][4], const T* __restrict__ W0, TO* __restrict__ out,
                                            int tp, int tq, int d, int f, float eta) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tq * kTile + acc_q(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = tp * kTile + acc_p(i, g);
        if (q < d && p < f) {
          const int64_t o = (int64_t)q * f + p;
          f32x4 w = load4(W0 + o);
          store4(out + o, fmaf(eta, acc[i][j][4 * g], w[0]), fmaf(eta, acc[i][j][4 * g + 1], w[1]),
                 fmaf(eta, acc[i][j][4 * g + 2], w[2]), fmaf(eta, acc[i][j][4 * g + 3], w[3]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounds the live W0 loads
    }
}

// Per-chunk delta dW[b, c] = V^_c^T Z_c (Method §3, step 1).  P = d_ff (Z
// columns), Q = d_model (V^ columns), K = the chunk's tokens; both operands are
// token-major, hence MN-contiguous.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_chunk_delta(const T* __restrict__ Z, const T* __restrict__ Vh,
                                                           float* __restrict__ dW, int B, int n, int d, int f, int C) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int TP = (f + kTile - 1) / kTile, TQ = (d + kTile - 1) / kTile;
  const int per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bc = id / per;
  int tp, tq;
  grouped_tile(id - bc * per, TP, TQ, 4, tp, tq);
  const int k = n / C;
  const int b = bc / k, c = bc - b * k;
  const int64_t row0 = (int64_t)b * n + (int64_t)c * C;

  LoadMC<T> lp, lq;
  lp.init(Z + row0 * f + tp * kTile, f, f - tp * kTile, C);
  lq.init(Vh + row0 * d + tq * kTile, d, d - tq * kTile, C);
  f32x16 acc[4][4];
  mainloop<T>(lp, lq, (C + LoadMC<T>::BK - 1) / LoadMC<T>::BK, acc, smem, NoHook{});

  float* out = dW + (int64_t)bc * d * f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tq * kTile + acc_q(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = tp * kTile + acc_p(i, g);
        if (q < d && p < f)
          store4(out + (int64_t)q * f + p, acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
      }
    }
}

// Exclusive prefix scan over chunks (Method §3, steps 2-3), four elements per
// thread: Wc[b, c] = W0 + eta * sum_{j<c} dW[b, j]; W_final = W0 + eta * sum_all.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_chunk_scan(const float* __restrict__ dW, const T* __restrict__ W0,
                                                          T* __restrict__ Wc, float* __restrict__ Wf, int k,
                                                          int64_t df, float eta) {
  const int64_t e = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  const int b = blockIdx.y;
  if (e >= df) return;
  const f32x4 w0 = load4(W0 + e);
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
  const float* src = dW + (int64_t)b * k * df + e;
  T* dst = Wc + (int64_t)b * k * df + e;
  for (int c = 0; c < k; ++c) {
    store4(dst + (int64_t)c * df, fmaf(eta, s[0], w0[0]), fmaf(eta, s[1], w0[1]), fmaf(eta, s[2], w0[2]),
           fmaf(eta, s[3], w0[3]));
    s += load4(src + (int64_t)c * df);
  }
  store4(Wf + (int64_t)b * df + e, fmaf(eta, s[0], w0[0]), fmaf(eta, s[1], w0[1]), fmaf(eta, s[2], w0[2]),
         fmaf(eta, s[3], w0[3]));
}

// Fused delta + scan: each workgroup owns one [256 d_model x 256 d_ff] tile of
// the state and runs its K loop over the whole sequence in token order; the
// accumulator is the running sum of the deltas, so at every chunk boundary it
// is exactly the exclusive prefix of the next chunk.
template <typename T>
struct SnapshotHook {
  const T* W0;
  T* Wc;              // [k, d, f] of this batch row
  int steps_per_chunk, k, tp, tq, d, f;
  float eta;
  __device__ __forceinline__ void operator()(int ks, f32x16 (&acc)[4][4]) const {
    const int done = ks + 1;
    if (done % steps_per_chunk != 0) return;
    const int c = done / steps_per_chunk;
    if (c >= k) return;
    write_state(acc, W0, Wc + (int64_t)c * d * f, tp, tq, d, f, eta);
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_chunk_update_scan(const T* __restrict__ Z, const T* __restrict__ Vh,
                                                                 const T* __restrict__ W0, T* __restrict__ Wc,
                                                                 float* __restrict__ Wf, int B, int n, int d, int f,
                                                                 int C, float eta) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int TP = (f + kTile - 1) / kTile, TQ = (d + kTile - 1) / kTile;
  const int per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per;
  int tp, tq;
  grouped_tile(id - b * per, TP, TQ, 4, tp, tq);
  const int k = n / C;
  const int64_t row0 = (int64_t)b * n;
  T* wc = Wc + (int64_t)b * k * d * f;

  LoadMC<T> lp, lq;
  lp.init(Z + row0 * f + tp * kTile, f, f - tp * kTile, n);
  lq.init(Vh + row0 * d + tq * kTile, d, d - tq * kTile, n);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  write_state(acc, W0, wc, tp, tq, d, f, 0.f);                        // chunk 0: W_down0
  SnapshotHook<T> hook{W0, wc, C / LoadMC<T>::BK, k, tp, tq, d, f, eta};
  mainloop<T>(lp, lq, n / LoadMC<T>::BK, acc, smem, hook);
  write_state(acc, W0, Wf + (int64_t)b * d * f, tp, tq, d, f, eta);  // after the last chunk
}

// ------------------------------------------------------------------ apply

// O_c = Z_c W^T for every chunk (eq. (3)).  P = d_model (rows of W), Q = the
// chunk's tokens, K = d_ff; both operands K-contiguous.  W of (b, c) is
// W + b * wsb + c * wsc.  With MSE, also R_c = O_c - V^_c into R [B, C, d].
template <typename T, bool MSE>
__global__ __launch_bounds__(kThreads) void k_apply(const T* __restrict__ Z, const T* __restrict__ W, int64_t wsb,
                                                     int64_t wsc, T* __restrict__ O, const T* __restrict__ Vh,
                                                     T* __restrict__ R, int n, int d, int f, int C, int nch,
                                                     int c_first) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int TP = (d + kTile - 1) / kTile, TQ = (C + kTile - 1) / kTile;
  const int per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bc = id / per;
  int tp, tq;
  grouped_tile(id - bc * per, TP, TQ, 4, tp, tq);
  const int b = bc / nch, c = c_first + (bc - b * nch);
  const T* Wbc = W + (int64_t)b * wsb + (int64_t)c * wsc;
  const int64_t row0 = (int64_t)b * n + (int64_t)c * C;

  LoadKC<T> lp, lq;
  lp.init([&](int r) -> const T* {
    int i = tp * kTile + r;
    return i < d ? Wbc + (int64_t)i * f : nullptr;
  }, f);
  lq.init([&](int r) -> const T* {
    int t = tq * kTile + r;
    return t < C ? Z + (row0 + t) * f : nullptr;
  }, f);
  f32x16 acc[4][4];
  mainloop<T>(lp, lq, (f + LoadKC<T>::BK - 1) / LoadKC<T>::BK, acc, smem, NoHook{});

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tq * kTile + acc_q(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = tp * kTile + acc_p(i, g);
        if (t < C && p < d) {
          const int64_t o = (row0 + t) * d + p;
          store4(O + o, acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          if constexpr (MSE) {
            f32x4 v = load4(Vh + o);
            store4(R + ((int64_t)b * C + t) * d + p, acc[i][j][4 * g] - v[0], acc[i][j][4 * g + 1] - v[1],
                   acc[i][j][4 * g + 2] - v[2], acc[i][j][4 * g + 3] - v[3]);
          }
        }
      }
    }
}

// ------------------------------------------------------------------ MSE objective: state update

// W_{c+1} = W_c - (eta / C) R_c^T Z_c with R_c = Z_c W_c^T - V^_c (eq. (4) with
// the squared error at the pre-update state).  P = d_ff, Q = d_model, K = the
// chunk's tokens.  The fp32 state lives in Ws [B, d, f]; for c == 0 the previous
// state is W_down0.  Wsh (may be null) receives a dtype copy for the next apply.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_mse_update(const T* __restrict__ Z, const T* __restrict__ R,
                                                          const T* __restrict__ W0, float* __restrict__ Ws,
                                                          T* __restrict__ Wsh, int n, int d, int f, int C, int c,
                                                          float scale) {
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  const int TP = (f + kTile - 1) / kTile, TQ = (d + kTile - 1) / kTile;
  const int per = TP * TQ;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per;
  int tp, tq;
  grouped_tile(id - b * per, TP, TQ, 4, tp, tq);
  const int64_t row0 = (int64_t)b * n + (int64_t)c * C;

  LoadMC<T> lp, lq;
  lp.init(Z + row0 * f + tp * kTile, f, f - tp * kTile, C);
  lq.init(R + (int64_t)b * C * d + tq * kTile, d, d - tq * kTile, C);
  f32x16 acc[4][4];
  mainloop<T>(lp, lq, (C + LoadMC<T>::BK - 1) / LoadMC<T>::BK, acc, smem, NoHook{});

  float* ws = Ws + (int64_t)b * d * f;
  T* wsh = Wsh ? Wsh + (int64_t)b * d * f : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = tq * kTile + acc_q(j);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = tp * kTile + acc_p(i, g);
        if (q < d && p < f) {
          const int64_t o = (int64_t)q * f + p;
          f32x4 w = (c == 0) ? load4(W0 + o) : load4(ws + o);
          float nw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) nw[e] = fmaf(-scale, acc[i][j][4 * g + e], w[e]);
          store4(ws + o, nw[0], nw[1], nw[2], nw[3]);
          if (wsh) store4(wsh + o, nw[0], nw[1], nw[2], nw[3]);
        }
      }
    }
}

// ------------------------------------------------------------------ launchers

static inline unsigned grid1(int64_t tiles) { return (unsigned)tiles; }

template <typename T>
hipError_t launch_produce_z(const T* H, const T* Wg, const T* Wu, T* Z, int64_t rows, int d, int f, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  int64_t tiles = (int64_t)((f + 127) / 128) * ((rows + kTile - 1) / kTile);
  k_produce_z<T><<<grid1(tiles), kThreads, 0, s>>>(H, Wg, Wu, Z, rows, d, f);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_produce_vhat(const T* X0, const T* cw, const T* Wt, T* Vh, int64_t rows, int n, int d, int K,
                               hipStream_t s) {
  if (rows == 0) return hipSuccess;
  int64_t tiles = (int64_t)((d + kTile - 1) / kTile) * ((rows + kTile - 1) / kTile);
  dim3 g(grid1(tiles));
  switch (K) {
#define TTT_KW(KW) case KW: k_produce_vhat<T, KW><<<g, kThreads, 0, s>>>(X0, cw, Wt, Vh, rows, n, d); break;
    TTT_KW(1) TTT_KW(2) TTT_KW(3) TTT_KW(4) TTT_KW(5) TTT_KW(6) TTT_KW(7) TTT_KW(8)
#undef TTT_KW
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_chunk_delta(const T* Z, const T* Vh, float* dW, int B, int n, int d, int f, int C, hipStream_t s) {
  int64_t tiles = (int64_t)((f + kTile - 1) / kTile) * ((d + kTile - 1) / kTile) * B * (n / C);
  if (tiles == 0) return hipSuccess;
  k_chunk_delta<T><<<grid1(tiles), kThreads, 0, s>>>(Z, Vh, dW, B, n, d, f, C);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_chunk_scan(const float* dW, const T* W0, T* Wc, float* Wf, int B, int k, int64_t df, float eta,
                             hipStream_t s) {
  if (B == 0) return hipSuccess;
  dim3 g((unsigned)((df / 4 + kThreads - 1) / kThreads), (unsigned)B);
  k_chunk_scan<T><<<g, kThreads, 0, s>>>(dW, W0, Wc, Wf, k, df, eta);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_chunk_update_scan(const T* Z, const T* Vh, const T* W0, T* Wc, float* Wf, int B, int n, int d,
                                    int f, int C, float eta, hipStream_t s) {
  int64_t tiles = (int64_t)((f + kTile - 1) / kTile) * ((d + kTile - 1) / kTile) * B;
  if (tiles == 0) return hipSuccess;
  k_chunk_update_scan<T><<<grid1(tiles), kThreads, 0, s>>>(Z, Vh, W0, Wc, Wf, B, n, d, f, C, eta);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_apply(const T* Z, const T* W, int64_t wsb, int64_t wsc, T* O, int B, int n, int d, int f, int C,
                        hipStream_t s) {
  const int k = n / C;
  int64_t tiles = (int64_t)((d + kTile - 1) / kTile) * ((C + kTile - 1) / kTile) * B * k;
  if (tiles == 0) return hipSuccess;
  k_apply<T, false><<<grid1(tiles), kThreads, 0, s>>>(Z, W, wsb, wsc, O, nullptr, nullptr, n, d, f, C, k, 0);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mse_chunk(const T* Z, const T* Vh, const T* W0, const T* Wcur, float* Ws, T* Wsh, T* O, T* R, int B,
                            int n, int d, int f, int C, int c, float eta, hipStream_t s) {
  int64_t ta = (int64_t)((d + kTile - 1) / kTile) * ((C + kTile - 1) / kTile) * B;
  const int64_t df = (int64_t)d * f;
  // the state chunk c is applied with: W_down0 (shared) for c == 0, else this row's copy
  const T* W = (c == 0) ? W0 : Wcur;
  const int64_t wsb = (c == 0) ? 0 : df;
  k_apply<T, true><<<grid1(ta), kThreads, 0, s>>>(Z, W, wsb, 0, O, Vh, R, n, d, f, C, 1, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t tu = (int64_t)((f + kTile - 1) / kTile) * ((d + kTile - 1) / kTile) * B;
  k_mse_update<T><<<grid1(tu), kThreads, 0, s>>>(Z, R, W0, Ws, Wsh, n, d, f, C, c, eta / (float)C);
  return hipGetLastError();
}

#define TTT_INST(T)                                                                                               \
  template hipError_t launch_produce_z<T>(const T*, const T*, const T*, T*, int64_t, int, int, hipStream_t);     \
  template hipError_t launch_produce_vhat<T>(const T*, const T*, const T*, T*, int64_t, int, int, int,            \
                                             hipStream_t);                                                        \
  template hipError_t launch_chunk_delta<T>(const T*, const T*, float*, int, int, int, int, int, hipStream_t);   \
  template hipError_t launch_chunk_scan<T>(const float*, const T*, T*, float*, int, int, int64_t, float,         \
                                           hipStream_t);                                                          \
  template hipError_t launch_chunk_update_scan<T>(const T*, const T*, const T*, T*, float*, int, int, int, int,  \
                                                  int, float, hipStream_t);                                       \
  template hipError_t launch_apply<T>(const T*, const T*, int64_t, int64_t, T*, int, int, int, int, int,          \
                                      hipStream_t);                                                               \
  template hipError_t launch_mse_chunk<T>(const T*, const T*, const T*, const T*, float*, T*, T*, T*, int, int,  \
                                          int, int, int, int, float, hipStream_t);
TTT_INST(float)
TTT_INST(bf16)
#undef TTT_INST

}  // namespace ttt
