// Host-side launchers of the device kernels (internal to the library).
// Every launcher assumes its arguments were validated by the C ABI layer.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;

template <typename T>
hipError_t launch_conv(const T* X0, const T* cw, T* Y, int64_t rows, int n, int d, int K, hipStream_t s);
template <typename T>
hipError_t launch_transpose(const T* src, T* dst, int batch, int R, int C, float scale, hipStream_t s);
template <typename T>
hipError_t launch_produce_z(const T* H, const T* Wg, const T* Wu, T* Z, T* Zt, int64_t rows, int n, int d, int f,
                            hipStream_t s);
template <typename T>
hipError_t launch_produce_vhat(const T* Y, const T* WtT, T* Vt, int64_t rows, int n, int d, float scale,
                               hipStream_t s);
template <typename T>
hipError_t launch_chunk_delta(const T* Zt, const T* Vt, float* dW, int B, int n, int d, int f, int C, hipStream_t s);
template <typename T>
hipError_t launch_chunk_scan(const float* dW, const T* W0, T* Wc, float* Wf, int B, int k, int64_t df, float eta,
                             hipStream_t s);
template <typename T>
hipError_t launch_chunk_update_scan(const T* Zt, const T* Vt, const T* W0, T* Wc, float* Wf, T* Wp, float* Tot,
                                    int B, int n, int d, int f, int C, int S, hipStream_t s);

// Number of sequence segments the fused update-scan runs side by side: more
// than one only when it fills the 256 compute units markedly better with one
// batch row (a segment count must divide the chunk count).  It depends on the
// state's shape alone, so a batch row's summation order, and with it every
// bit of its result, does not depend on the other rows of the batch.
inline int update_scan_segments(int64_t d, int64_t f, int64_t k) {
  const int64_t tiles = ((f + 255) / 256) * ((d + 255) / 256);
  auto fill = [](int64_t t) { return t == 0 ? 1.0 : (double)t / (256.0 * (double)((t + 255) / 256)); };
  int S = 1;
  for (int cand : {2, 4})
    if (k % cand == 0 && fill(tiles * cand) > fill(tiles * S) + 0.05) S = cand;
  return S;
}
template <typename T>
hipError_t launch_apply(const T* Zt, const T* W, int64_t wsb, int64_t wsc, T* O, int B, int n, int d, int f, int C,
                        hipStream_t s);
template <typename T>
hipError_t launch_mse_chunk(const T* Zt, const T* Vt, const T* W0, const T* Wcur, float* Ws, T* Wsh, T* O,
                            T* Rt, int B, int n, int d, int f, int C, int c, float eta, hipStream_t s);

// LaCT SwiGLU fast weight (one call runs every chunk of every (batch, head)).
struct LactArgs {
  int B, H, n, dh, m, C, order;
  float eta;
  const void *q, *k, *v, *W1, *W3, *W2;
  void* O;
  float *W1f, *W3f, *W2f;
  char* ws;
};
template <typename T>
size_t lact_workspace_bytes(int B, int H, int n, int dh, int m, int C);
template <typename T>
hipError_t launch_lact(const LactArgs& a, hipStream_t s);

}  // namespace ttt
