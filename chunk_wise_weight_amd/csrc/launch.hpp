// Host-side launchers of the device kernels (internal to the library).
// Every launcher assumes its arguments were validated by the C ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;

template <typename T>
hipError_t launch_conv(const T* X0, const T* cw, T* Y, int64_t rows, int n, int d, int K, const uint8_t* docs, int C,
                       bool fwd, const T* halo, hipStream_t s);
template <typename T>
// umask (with chunk > 0): rows of chunks whose update flag [batch, R / chunk]
// is zero are scaled by zero.
hipError_t launch_transpose(const T* src, T* dst, int batch, int R, int C, float scale, int rev, hipStream_t s,
                            const uint8_t* umask = nullptr, int chunk = 0);
template <typename T>
hipError_t launch_produce_z(const T* H, const T* Wg, const T* Wu, T* Z, T* Zt, int64_t rows, int n, int d, int f,
                            hipStream_t s);
template <typename T>
hipError_t launch_produce_vhat(const T* Y, const T* WtT, T* Vt, int64_t rows, int n, int d, float scale,
                               hipStream_t s, const uint8_t* umask = nullptr, int C = 0);
template <typename T>
hipError_t launch_chunk_delta(const T* Zt, const T* Vt, float* dW, int B, int n, int d, int f, int C, hipStream_t s);
template <typename T>
hipError_t launch_chunk_scan(const float* dW, const T* W0, T* Wc, float* Wf, int B, int k, int64_t df, float eta,
                             const uint8_t* docs, const float* Winit, hipStream_t s, bool inclusive = false);
// Operand layouts of the fused update-scan: the token-contiguous copies Zt
// [B, f, n] and Vt [B, d, n]; Z [B, n, f] and V [B, n, d] as they are; the
// latter with the chunks scanned last to first.  inclusive (token-contiguous
// layout, S <= 2): Wc[b, c] is the state after chunk c's own step, W_{c+1}
// (the update-then-apply order), and no initial state is written.
constexpr int kScanTokenContiguous = 0, kScanRowMajor = 1, kScanRowMajorReversed = 2;
template <typename T>
hipError_t launch_chunk_update_scan(const T* Zt, const T* Vt, const T* W0, T* Wc, float* Wf, T* Wp, float* Tot,
                                    int B, int n, int d, int f, int C, int S, const uint8_t* docs, const float* Winit,
                                    hipStream_t s, int layout = kScanTokenContiguous, bool inclusive = false);

// Number of sequence segments the fused update-scan runs side by side (a
// segment count divides the chunk count), by a two-term cost model: the K loop
// takes ceil(tiles S / 256) rounds of k C / S tokens at about 28 ns per token
// and round, and with four segments the fix-up pass reads and writes the
// (k - k / S) partial states of the later segments, 4 bytes per state element
// at about 5.5 TB/s.  Two segments are chained instead (the second takes the
// first's end state one chunk into its K loop, no partial states): no fix-up,
// but at least two rounds, since a second-segment tile that runs beside its
// partner waits for it.  Both rates are measured on the 128K workload (2560 x
// 9728 state, 380 tiles): two chained segments give three rounds of
// half-length tiles against two of full length.  The count depends on the
// state's and the sequence's shape alone, so a batch row's summation order,
// and with it every bit of its result, does not depend on the other rows of
// the batch.
inline int update_scan_segments(int64_t d, int64_t f, int64_t k, int64_t C) {
  const int64_t tiles = ((f + 255) / 256) * ((d + 255) / 256);
  auto cost = [&](int64_t S) {
    const int64_t r = (tiles * S + 255) / 256;
    const double rounds = (double)(S == 2 && r < 2 ? 2 : r);
    const double fixup = S > 2 ? (double)(k - k / S) * (double)(d * f) * 4.0 / 5.5e12 : 0.0;
    return rounds * (double)(k * C / S) * 28.1e-9 + fixup;
  };
  int S = 1;
  for (int cand : {2, 4})
    if (k % cand == 0 && cost(cand) < cost(S)) S = cand;
  return S;
}
// znat: Zt is Z [B, n, f] row-major instead of the token-contiguous copy.
template <typename T>
hipError_t launch_apply(const T* Zt, const T* W, int64_t wsb, int64_t wsc, T* O, int B, int n, int d, int f, int C,
                        float oscale, hipStream_t s, bool znat = false);
// rd [B, k]: the document starts of the reversed chunk order (see k_rev_docs).
hipError_t launch_rev_docs(const uint8_t* docs, uint8_t* rd, int B, int k, hipStream_t s);
// dst [n] = scale * src (n % 4 == 0); with umask [B, k] the elements are [B, ntok, row] token rows of chunks of C
// tokens, and the rows of masked chunks become zero.
template <typename T>
hipError_t launch_scale(const T* src, T* dst, int64_t n, float scale, hipStream_t s, const uint8_t* umask = nullptr,
                        int row = 4, int ntok = 1, int C = 1);
// dZ_c = dO_c W_c + V_c S_c per chunk, V = eta V^ (backward of the dot chunk
// loop); states W_c at W + b wsb + c wsc and S_c at S + b ssb + c ssc, [d, f].
// The rows of V and dO are ldq elements apart (0: d).
template <typename T>
hipError_t launch_dz(const T* dO, const T* V, const T* W, int64_t wsb, int64_t wsc, const T* S, int64_t ssb,
                     int64_t ssc, T* dZ, int B, int n, int d, int f, int C, hipStream_t s, int ldq = 0);
// out [df] = sum over b of Tot [B rows, `stride` apart; stride 0: df] (fp32;
// df and stride multiples of 4).
hipError_t launch_sum_rows(const float* Tot, float* out, int B, int64_t df, hipStream_t s, int64_t stride = 0);
// The MSE loop's backward, one chunk c at a time: dZ_c = Tt^T W + Rt^T S with
// Tt, Rt one chunk's token-contiguous [B, d, C] buffers, W at W + b wsb and S
// at S + b ssb ([d, f] each).
template <typename T>
hipError_t launch_dz_chunk(const T* Tt, const T* Rt, const T* W, int64_t wsb, const T* S, int64_t ssb, T* dZ, int B,
                           int n, int d, int f, int C, int c, hipStream_t s);
// (launch_mse_chunk with znat, and the two below: Zt is Z [B, n, f] as it is.)
// The MSE apply alone for chunk c: Rt = rscale (O - V^)^T, or with gen
// rscale O^T + vscale V^T and O (if not null) scaled by oscale; the state is
// W_down0 at chunk 0 unless cont, else Wcur + b d f.
// Row b's state is Wcur + b wstride (0: d f).
template <typename T>
// umask [B, k] (or null): a masked chunk's rscale (and, with gen, oscale) is zero.
hipError_t launch_mse_apply_gen(const T* Zt, const T* Vt, const T* W0, const T* Wcur, T* O, T* Rt, bool cont, int B,
                                int n, int d, int f, int C, int c, float rscale, float vscale, float oscale, bool gen,
                                hipStream_t s, int64_t wstride = 0, const uint8_t* umask = nullptr);
// MSE backward, packed rows: where chunk c starts row b's document, dW0 += G[b] (rows in order) and G[b] (and
// Gsh[b]) = 0.  With dWi (resumed rows, c = 0): a row whose chunk 0 is not flagged continues from W_init, so
// dWi[b] = G[b] and dW0 takes nothing of it; flagged rows get dWi[b] = 0.
template <typename T>
hipError_t launch_doc_grad_reset(float* G, T* Gsh, float* dW0, const uint8_t* docs, int B, int k, int c, int64_t df,
                                 hipStream_t s, float* dWi = nullptr);
// Dot backward, resumed rows: Tt [B, d, f] the rows' first-document gradients; dWi[b] = Tt[b] where row b
// continues from W_init (chunk 0 not flagged), else 0; dW0 -= their sum (have_dW0: dW0 holds every document's
// sum), else dW0 = 0.
hipError_t launch_resume_split(const float* Tt, const uint8_t* docs, float* dW0, float* dWi, int B, int k, int64_t df,
                               bool have_dW0, hipStream_t s);
// Ws [B, k, d, f]: slot c gets the state the MSE apply of chunk c reads (W_down0
// where a document starts, else Wcur [B, d, f]).
template <typename T>
hipError_t launch_keep_state(const T* W0, const T* Wcur, T* Ws, const uint8_t* docs, bool cont, int B, int k, int c,
                             int64_t df, hipStream_t s);
// The MSE update alone: Ws (and Wsh) = Ws + Rt Z_c, seeded from W_down0 at chunk 0 unless cont.
template <typename T>
hipError_t launch_mse_update(const T* Zt, const T* Rt, const T* W0, float* Ws, T* Wsh, bool cont, int B, int n, int d,
                             int f, int C, int c, hipStream_t s);
// Backward of the producer: G [rows, 2f] = [dA | dU] from dZ [rows, f],
// recomputing A = H W_gate^T and U = H W_up^T.
template <typename T>
hipError_t launch_produce_z_bwd(const T* H, const T* Wg, const T* Wu, const T* dZ, T* G, int64_t rows, int n, int d,
                                int f, hipStream_t s);
// Backward of the causal convolution (fwd: of the forward-looking in-chunk one): dX0 [rows, d] and the
// tap-gradient partials part [conv_bwd_partials(rows), d, K] (fp32); with halo [B, K-1, d] (resumed rows, causal
// only) the first document of a row not flagged at chunk 0 reads it, and dhalo [B, K-1, d] (if not null) gets
// its gradient (zero for flagged rows and with fwd).
template <typename T>
hipError_t launch_conv_bwd(const T* X0, const T* cw, const T* dY, T* dX0, float* part, int64_t rows, int n, int d,
                           int K, hipStream_t s, const uint8_t* docs, int C, bool fwd = false,
                           const T* halo = nullptr, T* dhalo = nullptr);
// Number of tap-gradient partials launch_conv_bwd writes: a thread takes
// kConvBwdGroups groups of kConvBwdRows rows of one channel chunk.
constexpr int kConvBwdRows = 8, kConvBwdGroups = 32;
__host__ __device__ inline int64_t conv_bwd_partials(int64_t rows) {
  return (rows / kConvBwdRows + kConvBwdGroups - 1) / kConvBwdGroups;
}
// p [n] = 0 (n % 4 == 0).
template <typename T>
hipError_t launch_zero(T* p, int64_t n, hipStream_t s);
template <typename T>
hipError_t launch_mse_apply_state(const T* Zt, const T* Wcur, T* O, int B, int n, int d, int f, int Cs, int c,
                                  hipStream_t s);
template <typename T>
hipError_t launch_mse_chunk(const T* Zt, const T* Vt, const T* W0, const T* Wcur, float* Ws, T* Wsh, T* O,
                            T* Rt, const uint8_t* docs, bool cont, int B, int n, int d, int f, int C, int c,
                            float eta, hipStream_t s, const uint8_t* umask = nullptr, bool znat = false);
template <typename T>
hipError_t launch_state_copy(const float* Winit, float* Wf, T* Wsh, int B, int64_t df, hipStream_t s);

// LaCT SwiGLU fast weight (one call runs every chunk of every (batch, head)).
struct LactArgs {
  int B, H, n, dh, m, C, order;
  float eta;
  const void *q, *k, *v, *W1, *W3, *W2;
  void* O;
  float *W1f, *W3f, *W2f;
  char* ws;
  const unsigned char* update_mask;   // HOST [n / C]: chunks whose keys update the weights; null = every chunk
  const float* eta_tok;               // DEVICE [B, H, n] per-token learning rates, or null
  int loss_dot;                       // 1: dot-product loss -f(k)^T v; 0: squared error
  int weight_norm;                    // 1: L2-normalise the rows of W1, W3, W2 after every update
  int muon;                           // 1: step along Muon(g) (Newton-Schulz) instead of g
  hipStream_t side;                   // caller's side stream for the second row group, or null: one chain
  hipEvent_t fork, join;              // caller's events ordering the side stream's work within the call
  // backward's recompute: keys only (no query is applied, O is not written), and every state kept:
  // keep [k + 1, B H, 3, m dh] dtype, slot c = the operand copies (W1, W3, W2) before chunk c's update
  int keys_only;
  void* keep;
};
template <typename T>
size_t lact_bwd_workspace_bytes(int B, int H, int n, int dh, int m, int C, bool saved = false);
// Backward of the LaCT layer (squared error, plain GD, no other variant): dq, dk, dv [B, H, n, dh] dtype and the
// initial weights' gradients dW1, dW3 [H, m, dh], dW2 [H, dh, m] fp32, given dO; every state recomputed first.
struct LactBwdArgs {
  int B, H, n, dh, m, C, order;
  float eta;
  const void *q, *k, *v, *W1, *W3, *W2, *dO;
  void *dq, *dk, *dv;
  float *dW1, *dW3, *dW2;
  char* ws;
  const unsigned char* update_mask;   // HOST [n / C] as in LactArgs, or null
  const void* states;                 // the states the forward call kept (LactArgs::keep's layout), or null
};
template <typename T>
hipError_t launch_lact_backward(const LactBwdArgs& a, hipStream_t s);
// The forward's key-side kernels on one chunk's rows X (keys or queries of chunk c of [BH, n, dh]) with states W
// (row bh's W1, W3, W2 at W + bh wsb + 0, m dh, 2 m dh): A, U, Hh = silu(A) U [BH, C, m]; R = Hh W2^T - v
// [BH, C, dh] (v rows of chunk c of [BH, n, dh]).
template <typename T>
hipError_t launch_lact_gate_pass(const T* X, const T* W, int64_t wsb, T* A, T* U, T* Hh, int BH, int n, int dh,
                                 int m, int C, int c, hipStream_t s);
template <typename T>
hipError_t launch_lact_residual_pass(const T* Hh, const T* W, int64_t wsb, const T* v, T* R, int BH, int n, int dh,
                                     int m, int C, int c, hipStream_t s);
template <typename T>
size_t lact_workspace_bytes(int B, int H, int n, int dh, int m, int C);
template <typename T>
hipError_t launch_lact(const LactArgs& a, hipStream_t s);

}  // namespace ttt
