// C ABI of the chunk-wise TTT library: argument validation (always complete
// before any device work), workspace planning and dispatch to the launchers.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "ttt.h"

namespace {

using ttt::bf16;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }

// Steps of the bf16 / fp32 K loop: the fused update-scan needs chunk
// boundaries on step boundaries.
inline int64_t kstep(int dtype) { return dtype == TTT_BF16 ? 64 : 32; }

struct Plan {
  int mode;
  int64_t B, n, d, f, C, K, k;
  size_t esz;
  bool fused;
  int S;              // sequence segments of the fused update-scan
  // workspace regions (byte offsets); Y and WtT only with the producers
  size_t off_Y, off_WtT, off_Zt, off_Vt, off_Wc, off_dW, off_Wp, off_Tot, off_Rt, off_Wsh, total;
  const uint8_t* docs;  // document starts [B, k] (device) or null: one document per batch row
  bool conv_fwd;        // forward-looking in-chunk convolution for the target
  const float* Winit;   // resumed rows: state before chunk 0 [B, d, f] fp32 (device) or null
  const void* halo;     // resumed rows: X0 rows before the first token [B, K-1, d] (device) or null
  void* states;         // dot objective: where the per-chunk states go [B, k, d, f] (device), or null: workspace
  const uint8_t* umask; // update mask [B, k] (device) or null: every chunk updates
  bool update_first;    // each chunk's step before its apply
};

int check_inplace_shape(const ttt_inplace_shape* s, int dtype) {
  if (s == nullptr) return TTT_ERR_ARG;
  if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_ERR_DTYPE;
  if (s->batch < 0 || s->seq_len < 0 || s->d_model <= 0 || s->d_ff <= 0 || s->chunk <= 0 || s->conv_k <= 0)
    return TTT_ERR_SHAPE;
  if (s->seq_len % s->chunk != 0) return TTT_ERR_SHAPE;
  if (s->d_model % 8 || s->d_ff % 8 || s->chunk % 8 || s->conv_k > 8) return TTT_ERR_UNSUPPORTED;
  // index, buffer-offset and grid ranges the kernels are built for
  const int64_t lim = (int64_t)1 << 30;
  if (s->d_model > (1 << 16) || s->d_ff > (1 << 20) || s->seq_len > ((int64_t)1 << 22) || s->batch > lim ||
      s->batch * s->seq_len > lim)
    return TTT_ERR_UNSUPPORTED;
  const int64_t rows_tiles = (s->batch * s->seq_len + 255) / 256;
  if (rows_tiles * ((s->d_ff + 127) / 128) > INT32_MAX) return TTT_ERR_UNSUPPORTED;
  const int64_t k = s->seq_len / s->chunk;
  if (s->batch * k * ((s->d_model + 255) / 256) * ((s->d_ff + 255) / 256) > INT32_MAX) return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}

int make_plan(const ttt_inplace_shape* s, int dtype, int mode, bool producers, Plan* p) {
  int st = check_inplace_shape(s, dtype);
  if (st != TTT_OK) return st;
  if (mode != TTT_MODE_DOT && mode != TTT_MODE_MSE && mode != TTT_MODE_DOT_SCAN) return TTT_ERR_ARG;
  p->docs = nullptr;
  p->conv_fwd = false;
  p->Winit = nullptr;
  p->halo = nullptr;
  p->states = nullptr;
  p->umask = nullptr;
  p->update_first = false;
  p->mode = mode;
  p->B = s->batch;
  p->n = s->seq_len;
  p->d = s->d_model;
  p->f = s->d_ff;
  p->C = s->chunk;
  p->K = s->conv_k;
  p->k = s->seq_len / s->chunk;
  p->esz = dtype == TTT_BF16 ? 2 : 4;
  p->fused = mode == TTT_MODE_DOT && p->C % kstep(dtype) == 0;
  const size_t BN = (size_t)p->B * p->n, DF = (size_t)p->d * p->f;
  size_t off = 0;
  p->S = p->fused ? ttt::update_scan_segments(p->d, p->f, p->k, p->C) : 1;
  p->off_Y = p->off_WtT = p->off_Zt = p->off_Vt = p->off_Wc = p->off_dW = p->off_Wp = p->off_Tot = 0;
  p->off_Rt = p->off_Wsh = 0;
  if (producers) {
    p->off_Y = off;
    off += align_up(BN * p->d * p->esz);
    p->off_WtT = off;
    off += align_up((size_t)p->d * p->d * p->esz);
  }
  p->off_Zt = off;
  off += align_up(BN * p->f * p->esz);
  p->off_Vt = off;
  off += align_up(BN * p->d * p->esz);
  if (mode == TTT_MODE_DOT || mode == TTT_MODE_DOT_SCAN) {
    p->off_Wc = off;
    off += align_up((size_t)p->B * p->k * DF * p->esz);
    if (!p->fused) {
      p->off_dW = off;
      off += align_up((size_t)p->B * p->k * DF * 4);
    } else if (p->S > 1) {
      p->off_Wp = off;
      off += align_up((size_t)p->B * (p->k - p->k / p->S) * DF * p->esz);
      p->off_Tot = off;
      off += align_up((size_t)p->B * (p->S - 1) * DF * 4);
    }
  } else {
    p->off_Rt = off;
    off += align_up((size_t)p->B * p->C * p->d * p->esz);
    if (dtype == TTT_BF16) {
      p->off_Wsh = off;
      off += align_up((size_t)p->B * DF * p->esz);
    }
  }
  p->total = off;
  return TTT_OK;
}

inline int dev(hipError_t e) { return e == hipSuccess ? TTT_OK : TTT_ERR_DEVICE; }

// W_final[b] = W_down0 (a resumed row: its own state) for every row (no
// chunks): the scan with zero chunks.
template <typename T>
int fill_initial_state(const Plan& p, const void* W0, float* Wf, hipStream_t s) {
  return dev(ttt::launch_chunk_scan<T>(nullptr, (const T*)W0, nullptr, Wf, (int)p.B, 0, (int64_t)p.d * p.f, 0.f, nullptr,
                                       p.Winit, s));
}

// Scale the target is produced with: the fused dot update takes eta folded
// into the target (eta V^_c^T Z_c = (eta V^_c)^T Z_c), every other plan takes V^.
inline float target_scale(const Plan& p, int mode, float eta) {
  return (mode == TTT_MODE_DOT && p.fused) ? eta : 1.0f;
}

// The chunk loop, given the token-contiguous Zt [B, f, n] and Vt [B, d, n] (Vt
// scaled by target_scale).  Every contraction over f reads Zt as well, by
// transposing tiles in LDS, so no row-major Z is needed.
template <typename T>
int run_core(const Plan& p, int mode, float eta, const void* Ztv, const void* Vtv, const void* W0v, void* Ov,
             float* Wf, char* ws, hipStream_t s) {
  const T* Zt = (const T*)Ztv;
  const T* Vt = (const T*)Vtv;
  const T* W0 = (const T*)W0v;
  T* O = (T*)Ov;
  const int B = (int)p.B, n = (int)p.n, d = (int)p.d, f = (int)p.f, C = (int)p.C, k = (int)p.k;
  const int64_t df = (int64_t)d * f;
  if (p.B == 0) return TTT_OK;
  if (p.n == 0) return fill_initial_state<T>(p, W0v, Wf, s);
  if (mode == TTT_MODE_MSE) {
    T* Rt = (T*)(ws + p.off_Rt);
    T* Wsh = p.esz == 2 ? (T*)(ws + p.off_Wsh) : nullptr;
    const T* Wcur = p.esz == 2 ? (const T*)Wsh : (const T*)(const void*)Wf;
    if (p.Winit != nullptr) {      // resumed rows: the state and its operand copy start from W_init
      int st = dev(ttt::launch_state_copy<T>(p.Winit, Wf, Wsh, B, df, s));
      if (st != TTT_OK) return st;
    }
    for (int c = 0; c < k; ++c) {
      int st = TTT_OK;
      if (p.states != nullptr)      // the state this chunk's apply reads, kept for a backward pass
        st = dev(ttt::launch_keep_state<T>(W0, Wcur, (T*)p.states, p.docs, p.Winit != nullptr, B, k, c, df, s));
      if (st == TTT_OK)
        st = dev(ttt::launch_mse_chunk<T>(Zt, Vt, W0, Wcur, Wf, Wsh, p.update_first ? nullptr : O, Rt, p.docs,
                                          p.Winit != nullptr, B, n, d, f, C, c, eta, s, p.umask));
      // update first: the chunk applied again with the state its step left
      if (st == TTT_OK && p.update_first)
        st = dev(ttt::launch_mse_apply_state<T>(Zt, Wcur, O, B, n, d, f, C, c, s));
      if (st != TTT_OK) return st;
    }
    return TTT_OK;
  }
  T* Wc = p.states != nullptr ? (T*)p.states : (T*)(ws + p.off_Wc);
  int st;
  if (p.fused) {
    st = dev(ttt::launch_chunk_update_scan<T>(Zt, Vt, W0, Wc, Wf, (T*)(ws + p.off_Wp), (float*)(ws + p.off_Tot),
                                              B, n, d, f, C, p.S, p.docs, p.Winit, s, ttt::kScanTokenContiguous,
                                              p.update_first));   // Vt carries eta
  } else {
    float* dW = (float*)(ws + p.off_dW);
    st = dev(ttt::launch_chunk_delta<T>(Zt, Vt, dW, B, n, d, f, C, s));
    if (st == TTT_OK)
      st = dev(ttt::launch_chunk_scan<T>(dW, W0, Wc, Wf, B, k, df, eta, p.docs, p.Winit, s, p.update_first));
  }
  if (st != TTT_OK) return st;
  return dev(ttt::launch_apply<T>(Zt, Wc, (int64_t)k * df, df, O, B, n, d, f, C, 1.0f, s));
}

// Zt and Vt from the producers' inputs.
template <typename T>
int run_producers(const Plan& p, const void* H, const void* X0, const void* Wg, const void* Wu, const void* Wt,
                  const void* cw, char* ws, T* Zt, T* Vt, float vscale, hipStream_t s) {
  const int64_t rows = p.B * p.n;
  if (rows == 0) return TTT_OK;
  const int n = (int)p.n, d = (int)p.d, f = (int)p.f;
  T* Y = (T*)(ws + p.off_Y);
  T* WtT = (T*)(ws + p.off_WtT);
  int st = dev(ttt::launch_produce_z<T>((const T*)H, (const T*)Wg, (const T*)Wu, nullptr, Zt, rows, n, d, f, s));
  if (st == TTT_OK) st = dev(ttt::launch_conv<T>((const T*)X0, (const T*)cw, Y, rows, n, d, (int)p.K, p.docs, (int)p.C,
                                                  p.conv_fwd, (const T*)p.halo, s));
  if (st == TTT_OK) st = dev(ttt::launch_transpose<T>((const T*)Wt, WtT, 1, d, d, 1.0f, 0, s));
  // the dot plans zero the targets of chunks that do not update; MSE zeroes their residuals instead
  const uint8_t* um = p.mode == TTT_MODE_MSE ? nullptr : p.umask;
  if (st == TTT_OK) st = dev(ttt::launch_produce_vhat<T>(Y, WtT, Vt, rows, n, d, vscale, s, um, (int)p.C));
  return st;
}

// Options common to the layer and the chunk loop; `producers`: the target
// producer's options (conv_forward, x0_halo) apply.
int apply_options(Plan& p, int mode, const ttt_layer_options* o, bool producers) {
  if (o == nullptr) return TTT_OK;
  if (producers && o->conv_forward != 0 && o->conv_forward != 1) return TTT_ERR_ARG;
  if (o->update_first != 0 && o->update_first != 1) return TTT_ERR_ARG;
  if (o->update_first == 1 && o->W_states != nullptr) return TTT_ERR_UNSUPPORTED;
  p.update_first = o->update_first == 1;
  // the fused plan writes the states after each chunk's step with one or two (chained) segments; four fall back
  // to one (its workspace holds less than the four-segment plan's)
  if (p.update_first && p.fused && p.S > 2) p.S = 1;
  if ((o->W_init != nullptr && !ok_ptr(o->W_init)) || (producers && o->x0_halo != nullptr && !ok_ptr(o->x0_halo)) ||
      (o->W_states != nullptr && !ok_ptr(o->W_states)))
    return TTT_ERR_ARG;
  p.docs = o->doc_starts;
  p.Winit = o->W_init;
  p.states = o->W_states;
  p.umask = o->update_mask;
  if (producers) {
    p.conv_fwd = o->conv_forward == 1;
    p.halo = p.K > 1 ? o->x0_halo : nullptr;
  }
  return TTT_OK;
}

int check_ws(const Plan& p, void* ws, size_t bytes) {
  if (p.total == 0) return TTT_OK;
  if (ws == nullptr || !aligned16(ws) || bytes < p.total) return TTT_ERR_WORKSPACE;
  return TTT_OK;
}

inline bool finite(float x) { return isfinite(x); }

template <typename T>
int layer(const Plan& p, int mode, float eta, const void* H, const void* X0, const void* Wg, const void* Wu,
          const void* W0, const void* Wt, const void* cw, void* O, float* Wf, char* ws, hipStream_t s) {
  T* Zt = (T*)(ws + p.off_Zt);
  T* Vt = (T*)(ws + p.off_Vt);
  int st = run_producers<T>(p, H, X0, Wg, Wu, Wt, cw, ws, Zt, Vt, target_scale(p, mode, eta), s);
  if (st != TTT_OK) return st;
  return run_core<T>(p, mode, eta, Zt, Vt, W0, O, Wf, ws, s);
}

template <typename T>
int core(const Plan& p, int mode, float eta, const void* Z, const void* V, const void* W0, void* O, float* Wf,
         char* ws, hipStream_t s) {
  T* Zt = (T*)(ws + p.off_Zt);
  T* Vt = (T*)(ws + p.off_Vt);
  int st = dev(ttt::launch_transpose<T>((const T*)Z, Zt, (int)p.B, (int)p.n, (int)p.f, 1.0f, 0, s));
  if (st == TTT_OK)
    st = dev(ttt::launch_transpose<T>((const T*)V, Vt, (int)p.B, (int)p.n, (int)p.d, target_scale(p, mode, eta), 0,
                                      s, mode == TTT_MODE_MSE ? nullptr : p.umask, (int)p.C));
  if (st != TTT_OK) return st;
  return run_core<T>(p, mode, eta, Zt, Vt, W0, O, Wf, ws, s);
}

// ------------------------------------------------------------------ backward of the dot chunk loop

// Workspace of ttt_core_backward: the recomputed states W_c and the suffix
// states S (in reverse chunk order), the rows' totals, a zero [d, f] start
// state, eta V^ (row-major, for dZ), and the scans' operands and scratch.  The
// fused scan reads Z, eta V^ and dO in their own layout and keeps segment
// partials; with a chunk length that does not suit it, the per-chunk deltas
// read token-contiguous copies (Z and V^ in order, Z and dO in reverse chunk
// order) and are kept in fp32.
struct BwdPlan {
  int64_t B, n, d, f, C, k;
  size_t esz;
  bool fused;
  bool saved;         // the states come from the caller
  const uint8_t* docs;  // document starts [B, k] (device) or null
  const uint8_t* umask; // update mask [B, k] (device) or null: every chunk updates
  const float* Winit;   // resumed rows: the initial states [B, d, f] fp32, or null
  float* dWi;           // their gradient [B, d, f] fp32 (with Winit)
  int S;
  size_t off_Zt, off_Vt, off_Vs, off_Zr, off_Gr, off_Wc, off_Sr, off_T, off_zero, off_Wp, off_Tot, off_dW, off_rd,
      total;
};

int make_bwd_plan(const ttt_inplace_shape* s, int dtype, bool saved, BwdPlan* p, bool docs = false) {
  int st = check_inplace_shape(s, dtype);
  if (st != TTT_OK) return st;
  memset(p, 0, sizeof(*p));
  p->saved = saved;
  p->B = s->batch;
  p->n = s->seq_len;
  p->d = s->d_model;
  p->f = s->d_ff;
  p->C = s->chunk;
  p->k = s->seq_len / s->chunk;
  p->esz = dtype == TTT_BF16 ? 2 : 4;
  p->fused = p->C % kstep(dtype) == 0;
  p->S = p->fused ? ttt::update_scan_segments(p->d, p->f, p->k, p->C) : 1;
  if (p->B * p->n == 0) return TTT_OK;      // nothing but a zero dW_down0
  const size_t BN = (size_t)p->B * p->n, DF = (size_t)p->d * p->f, BK = (size_t)p->B * p->k;
  size_t off = 0;
  auto take = [&](size_t* o, size_t bytes) {
    *o = off;
    off += align_up(bytes);
  };
  take(&p->off_Vs, BN * p->d * p->esz);
  if (!p->fused) {
    take(&p->off_Vt, BN * p->d * p->esz);
    take(&p->off_Zt, BN * p->f * p->esz);
    take(&p->off_Zr, BN * p->f * p->esz);
    take(&p->off_Gr, BN * p->d * p->esz);
  }
  if (!saved) take(&p->off_Wc, BK * DF * p->esz);
  take(&p->off_Sr, BK * DF * p->esz);
  take(&p->off_T, (size_t)p->B * DF * 4);
  take(&p->off_zero, DF * p->esz);
  if (p->fused && p->S > 1) {
    take(&p->off_Wp, (size_t)p->B * (p->k - p->k / p->S) * DF * p->esz);
    take(&p->off_Tot, (size_t)p->B * (p->S - 1) * DF * 4);
  } else if (!p->fused) {
    take(&p->off_dW, BK * DF * 4);
  }
  if (docs) take(&p->off_rd, BK);
  p->total = off;
  return TTT_OK;
}

// One exclusive scan over the chunks from W0 into the states Wc and the total
// Wf: the fused update-scan on row-major Z [B, n, f] and V [B, n, d] (V scaled
// by eta already), in chunk order or reversed; or deltas of the
// token-contiguous copies (in the order wanted) and a scan with eta.
template <typename T>
int bwd_scan(const BwdPlan& p, const T* Zt, const T* Vt, const T* W0, T* Wc, float* Wf, float eta, bool rev,
             char* ws, hipStream_t s, const uint8_t* docs = nullptr, const float* Winit = nullptr) {
  const int B = (int)p.B, n = (int)p.n, d = (int)p.d, f = (int)p.f, C = (int)p.C, k = (int)p.k;
  if (p.fused)
    return dev(ttt::launch_chunk_update_scan<T>(Zt, Vt, W0, Wc, Wf, (T*)(ws + p.off_Wp), (float*)(ws + p.off_Tot), B,
                                                n, d, f, C, p.S, docs, Winit, s,
                                                rev ? ttt::kScanRowMajorReversed : ttt::kScanRowMajor));
  float* dW = (float*)(ws + p.off_dW);
  int st = dev(ttt::launch_chunk_delta<T>(Zt, Vt, dW, B, n, d, f, C, s));
  if (st == TTT_OK) st = dev(ttt::launch_chunk_scan<T>(dW, W0, Wc, Wf, B, k, (int64_t)d * f, eta, docs, Winit, s));
  return st;
}

// The backward pass: both scans, then dV^ as an apply of the suffix states (in
// reverse chunk order, by a negative state stride) and dZ from both state
// sequences, and dW_down0 as the sum of the rows' totals.  Resumed rows
// (p.Winit): the states start from W_init, and the reversed scan's totals --
// each row's first-document gradient -- are the rows' dW_init, taken off
// dW_down0 where the row continues.
template <typename T>
int core_backward(const BwdPlan& p, float eta, const void* Zv, const void* Vv, const void* W0, const void* dOv,
                  const void* Wsaved, void* dZ, void* dV, float* dW0, char* ws, hipStream_t s, bool vs_ready = false) {
  const int B = (int)p.B, n = (int)p.n, d = (int)p.d, f = (int)p.f, C = (int)p.C, k = (int)p.k;
  const int64_t df = (int64_t)d * f;
  if (p.B * p.n == 0) {
    int st = dev(ttt::launch_zero<float>(dW0, df, s));
    if (st == TTT_OK && p.Winit != nullptr) st = dev(ttt::launch_zero<float>(p.dWi, p.B * df, s));
    return st;
  }
  const T* Z = (const T*)Zv;
  const T* V = (const T*)Vv;
  const T* dO = (const T*)dOv;
  T* Vs = (T*)(ws + p.off_Vs);     // eta V^ [B, n, d]
  T* Wc = p.saved ? (T*)Wsaved : (T*)(ws + p.off_Wc);
  T* Sr = (T*)(ws + p.off_Sr);
  T* Z0 = (T*)(ws + p.off_zero);
  float* Tt = (float*)(ws + p.off_T);
  const T* Slast = Sr + (int64_t)(k - 1) * df;      // S_c = Sr[k - 1 - c]: stride -df from here
  int st = dev(ttt::launch_zero<T>(Z0, df, s));
  // eta V^ with the targets of masked chunks zero (they add nothing to the states, so they get no gradient)
  if (st == TTT_OK && !vs_ready) st = dev(ttt::launch_scale<T>(V, Vs, (int64_t)B * n * d, eta, s, p.umask, d, n, C));
  if (st == TTT_OK && vs_ready && p.umask != nullptr)
    st = dev(ttt::launch_scale<T>(Vs, Vs, (int64_t)B * n * d, 1.0f, s, p.umask, d, n, C));
  // with packed documents the suffixes restart at each document's end (the reversed order's starts), and
  // dW_down0, every document's sum, comes from a contraction over all chunks (into Sr and Tt, before the suffixes)
  const uint8_t* rd = p.docs != nullptr ? (const uint8_t*)(ws + p.off_rd) : nullptr;
  if (st == TTT_OK && rd != nullptr) st = dev(ttt::launch_rev_docs(p.docs, (uint8_t*)rd, B, k, s));
  if (p.fused) {
    // W_c (its W_final lands in Tt and is overwritten by the scans after it)
    if (st == TTT_OK && !p.saved)
      st = bwd_scan<T>(p, Z, Vs, (const T*)W0, Wc, Tt, eta, false, ws, s, p.docs, p.Winit);
    if (st == TTT_OK && rd != nullptr) {
      st = bwd_scan<T>(p, Z, dO, Z0, Sr, Tt, 1.0f, false, ws, s);
      if (st == TTT_OK) st = dev(ttt::launch_sum_rows(Tt, dW0, B, df, s));
    }
    // last chunk first: Sr[t] = sum of dO_c^T Z_c over the chunks c > k - 1 - t (of the same document); Tt = all
    if (st == TTT_OK) st = bwd_scan<T>(p, Z, dO, Z0, Sr, Tt, 1.0f, true, ws, s, rd);
    if (st == TTT_OK)
      st = dev(ttt::launch_apply<T>(Z, Slast, (int64_t)k * df, -df, (T*)dV, B, n, d, f, C, eta, s, true));
  } else {
    T* Zt = (T*)(ws + p.off_Zt);
    T* Vt = (T*)(ws + p.off_Vt);
    T* Zr = (T*)(ws + p.off_Zr);
    T* Gr = (T*)(ws + p.off_Gr);
    if (st == TTT_OK) st = dev(ttt::launch_transpose<T>(Z, Zt, B, n, f, 1.0f, 0, s));
    if (st == TTT_OK && !p.saved) st = dev(ttt::launch_transpose<T>(V, Vt, B, n, d, 1.0f, 0, s, p.umask, C));
    if (st == TTT_OK) st = dev(ttt::launch_transpose<T>(Z, Zr, B, n, f, 1.0f, C, s));
    if (st == TTT_OK) st = dev(ttt::launch_transpose<T>(dO, Gr, B, n, d, 1.0f, C, s));
    if (st == TTT_OK && !p.saved)
      st = bwd_scan<T>(p, Zt, Vt, (const T*)W0, Wc, Tt, eta, false, ws, s, p.docs, p.Winit);
    if (st == TTT_OK && rd != nullptr) {
      st = bwd_scan<T>(p, Zr, Gr, Z0, Sr, Tt, 1.0f, true, ws, s);
      if (st == TTT_OK) st = dev(ttt::launch_sum_rows(Tt, dW0, B, df, s));
    }
    if (st == TTT_OK) st = bwd_scan<T>(p, Zr, Gr, Z0, Sr, Tt, 1.0f, true, ws, s, rd);
    if (st == TTT_OK)
      st = dev(ttt::launch_apply<T>(Zt, Slast, (int64_t)k * df, -df, (T*)dV, B, n, d, f, C, eta, s));
  }
  if (st == TTT_OK && p.umask != nullptr)      // a masked chunk's target reaches no state: its gradient is zero
    st = dev(ttt::launch_scale<T>((const T*)dV, (T*)dV, (int64_t)B * n * d, 1.0f, s, p.umask, d, n, C));
  if (st == TTT_OK)
    st = dev(ttt::launch_dz<T>(dO, Vs, Wc, (int64_t)k * df, df, Slast, (int64_t)k * df, -df, (T*)dZ, B, n, d, f, C,
                               s));
  if (st == TTT_OK && p.Winit != nullptr)
    st = dev(ttt::launch_resume_split(Tt, p.docs, dW0, p.dWi, B, k, df, rd != nullptr, s));
  else if (st == TTT_OK && rd == nullptr)
    st = dev(ttt::launch_sum_rows(Tt, dW0, B, df, s));
  return st;
}

// ------------------------------------------------------------------ backward of the MSE chunk loop

// Workspace of ttt_core_backward_mse: token-contiguous V^ and dO (Z is read as
// it is), the state each chunk was applied with ([B, k, d, f], the layout of
// the forward call's kept states), the forward state and the state gradient
// (fp32, with bf16 operand copies), and one chunk's two residual buffers
// [B, d, C].  With packed documents the rows' gradients go straight into
// dW_down0 at each document start, so nothing more is needed.
struct MsePlan {
  int64_t B, n, d, f, C, k;
  size_t esz;
  const uint8_t* docs;  // document starts [B, k] (device) or null
  const uint8_t* umask; // update mask [B, k] (device) or null
  const float* Winit;   // resumed rows: the initial states [B, d, f] fp32, or null
  float* dWi;           // their gradient [B, d, f] fp32 (with Winit)
  size_t off_Vt, off_Gt, off_St, off_Ws, off_Wsh, off_G, off_Gsh, off_Rt, off_Tt, total;
};

int make_mse_plan(const ttt_inplace_shape* s, int dtype, MsePlan* p, bool saved = false) {
  int st = check_inplace_shape(s, dtype);
  if (st != TTT_OK) return st;
  *p = MsePlan{};
  p->B = s->batch;
  p->n = s->seq_len;
  p->d = s->d_model;
  p->f = s->d_ff;
  p->C = s->chunk;
  p->k = s->seq_len / s->chunk;
  p->esz = dtype == TTT_BF16 ? 2 : 4;
  if (p->B * p->n == 0) return TTT_OK;
  const size_t BN = (size_t)p->B * p->n, DF = (size_t)p->d * p->f, e = p->esz, B = (size_t)p->B;
  size_t off = 0;
  auto take = [&](size_t* o, size_t bytes) {
    *o = off;
    off += align_up(bytes);
  };
  take(&p->off_Vt, BN * p->d * e);
  take(&p->off_Gt, BN * p->d * e);
  if (!saved) {
    take(&p->off_St, (size_t)p->k * B * DF * e);
    take(&p->off_Ws, B * DF * 4);
  }
  take(&p->off_G, B * DF * 4);
  if (dtype == TTT_BF16) {
    if (!saved) take(&p->off_Wsh, B * DF * e);
    take(&p->off_Gsh, B * DF * e);
  }
  take(&p->off_Rt, B * p->d * p->C * e);
  take(&p->off_Tt, B * p->d * p->C * e);
  p->total = off;
  return TTT_OK;
}

template <typename T>
int mse_backward(const MsePlan& p, float eta, const void* Zv, const void* Vv, const void* W0v, const void* dOv,
                 const void* Wsaved, void* dZv, void* dVv, float* dW0, char* ws, hipStream_t s) {
  const int B = (int)p.B, n = (int)p.n, d = (int)p.d, f = (int)p.f, C = (int)p.C, k = (int)p.k;
  const int64_t df = (int64_t)d * f;
  const bool resume = p.Winit != nullptr;
  if (p.B * p.n == 0) {
    int st = dev(ttt::launch_zero<float>(dW0, df, s));
    if (st == TTT_OK && resume) st = dev(ttt::launch_zero<float>(p.dWi, p.B * df, s));
    return st;
  }
  const bool bf = sizeof(T) == 2;
  const T* W0 = (const T*)W0v;
  const T* Zt = (const T*)Zv;           // Z [B, n, f] as it is (the kernels' row-major operand forms)
  T* Vt = (T*)(ws + p.off_Vt);
  T* Gt = (T*)(ws + p.off_Gt);
  T* St = (T*)(ws + p.off_St);
  float* Ws = (float*)(ws + p.off_Ws);
  float* G = (float*)(ws + p.off_G);
  T* Wsh = bf ? (T*)(ws + p.off_Wsh) : nullptr;
  T* Gsh = bf ? (T*)(ws + p.off_Gsh) : nullptr;
  const T* Wcur = bf ? (const T*)Wsh : (const T*)(const void*)Ws;       // the state operand the applies read
  const T* Gop = bf ? (const T*)Gsh : (const T*)(const void*)G;
  T* Rt = (T*)(ws + p.off_Rt);
  T* Tt = (T*)(ws + p.off_Tt);
  const float a = eta / (float)C;
  int st = dev(ttt::launch_transpose<T>((const T*)Vv, Vt, B, n, d, 1.0f, 0, s));
  if (st == TTT_OK) st = dev(ttt::launch_transpose<T>((const T*)dOv, Gt, B, n, d, 1.0f, 0, s));
  // the forward scan again, keeping in St [B, k, d, f] the state each chunk's apply reads (W_down0 at a document
  // start, W_init where a resumed row continues), unless the forward call kept them the same way (Wsaved)
  if (st == TTT_OK && Wsaved == nullptr && resume) st = dev(ttt::launch_state_copy<T>(p.Winit, Ws, Wsh, B, df, s));
  for (int c = 0; c < k && st == TTT_OK && Wsaved == nullptr; ++c) {
    st = dev(ttt::launch_keep_state<T>(W0, Wcur, St, p.docs, resume, B, k, c, df, s));
    if (st == TTT_OK)
      st = dev(ttt::launch_mse_chunk<T>(Zt, Vt, W0, Wcur, Ws, Wsh, nullptr, Rt, p.docs, resume, B, n, d, f, C, c, eta,
                                        s, p.umask, true));
  }
  // the state gradient G = dLoss/dW_{c+1}, zero after the last chunk, taken back chunk by chunk
  if (st == TTT_OK) st = dev(ttt::launch_zero<float>(G, (int64_t)B * df, s));
  if (st == TTT_OK && bf) st = dev(ttt::launch_zero<T>(Gsh, (int64_t)B * df, s));
  // packed or resumed rows: every document's gradient is added into dW_down0 at its first chunk (a resumed row's
  // first document's goes to dW_init instead)
  if (st == TTT_OK && (p.docs != nullptr || resume)) st = dev(ttt::launch_zero<float>(dW0, df, s));
  const T* Sb = Wsaved != nullptr ? (const T*)Wsaved : (const T*)St;
  const int64_t wstride = (int64_t)k * df;
  for (int c = k - 1; c >= 0 && st == TTT_OK; --c) {
    const T* Wc = Sb + (int64_t)c * df;                     // row b's W_c at Wc + b k d f
    // Rt = -(eta/C) R_c^T, R_c = Z_c W_c^T - V^_c
    st = dev(ttt::launch_mse_apply_gen<T>(Zt, Vt, W0, Wc, nullptr, Rt, true, B, n, d, f, C, c, -a, 0.f, 1.f, false,
                                          s, wstride, p.umask));
    // Tt = T_c^T = (dO_c - (eta/C) Z_c G^T)^T, and dV^_c = (eta/C) Z_c G^T
    if (st == TTT_OK)
      st = dev(ttt::launch_mse_apply_gen<T>(Zt, Gt, W0, Gop, (T*)dVv, Tt, true, B, n, d, f, C, c, -a, 1.0f, a, true,
                                            s, 0, p.umask));
    // dZ_c = T_c W_c - (eta/C) R_c G
    if (st == TTT_OK)
      st = dev(ttt::launch_dz_chunk<T>(Tt, Rt, Wc, wstride, Gop, df, (T*)dZv, B, n, d, f, C, c, s));
    // G <- G + T_c^T Z_c = dLoss/dW_c
    if (st == TTT_OK) st = dev(ttt::launch_mse_update<T>(Zt, Tt, W0, G, Gsh, true, B, n, d, f, C, c, s));
    // packed rows: a document's first chunk hands its gradient to dW_down0, and the one before starts from zero
    if (st == TTT_OK && (p.docs != nullptr || (resume && c == 0)))
      st = dev(ttt::launch_doc_grad_reset<T>(G, Gsh, dW0, p.docs, B, k, c, df, s, resume ? p.dWi : nullptr));
  }
  // (with documents, chunk 0 starts every row's first one, so every gradient is in dW_down0 or dW_init by now)
  if (st == TTT_OK && p.docs == nullptr && !resume) st = dev(ttt::launch_sum_rows(G, dW0, B, df, s));
  return st;
}

// ------------------------------------------------------------------ backward of the whole dot layer

// Workspace of ttt_layer_backward: the recomputed Z and Y, W_target^T, the
// chunk loop's backward (its own plan, whose eta V^ region is filled here), dZ,
// dV^, G = [dA | dU], dY, the two token-contraction scans' scratch (sized for
// the larger state, [2f, d] or [d, d]), and the tap-gradient partials.
struct LayerBwdPlan {
  int mode;                     // TTT_MODE_DOT or TTT_MODE_MSE: the chunk loop differentiated
  bool conv_fwd;                // the forward-looking in-chunk convolution for the target
  const void* halo;             // resumed rows: X0's K-1 rows before the first token [B, K-1, d], or null
  void* dhalo;                  // their gradient (with halo)
  BwdPlan core;                 // its backward, dot objective
  MsePlan mcore;                // its backward, MSE objective
  int64_t B, n, d, f, C, K;
  size_t esz;
  int kk;                       // chunks the weight-gradient scans are cut into (their segments divide it)
  int S_gu, S_t;                // segments of the [dW_gate; dW_up] and dW_target scans
  int64_t DFm, npart;
  size_t off_Z, off_Y, off_WtT, off_V, off_dZ, off_dV, off_G, off_dY, off_wWc, off_wWp, off_wTot, off_wWf,
      off_wzero, off_part, off_core, total;
};

int make_layer_bwd_plan(const ttt_inplace_shape* s, int dtype, bool saved, LayerBwdPlan* p,
                        int mode = TTT_MODE_DOT) {
  *p = LayerBwdPlan{};
  p->mode = mode;
  int st = make_bwd_plan(s, dtype, saved, &p->core, true);
  if (st != TTT_OK) return st;
  if (!p->core.fused) return TTT_ERR_UNSUPPORTED;     // the weight gradients take the fused scan's token steps
  if (mode == TTT_MODE_MSE && (st = make_mse_plan(s, dtype, &p->mcore, saved)) != TTT_OK) return st;
  p->B = s->batch;
  p->n = s->seq_len;
  p->d = s->d_model;
  p->f = s->d_ff;
  p->C = s->chunk;
  p->K = s->conv_k;
  p->esz = p->core.esz;
  const int64_t ks = kstep(dtype);
  p->kk = p->n % (4 * ks) == 0 ? 4 : p->n % (2 * ks) == 0 ? 2 : 1;
  const int64_t Cw = p->kk > 0 ? p->n / p->kk : 0;
  p->S_gu = ttt::update_scan_segments(2 * p->f, p->d, p->kk, Cw);
  p->S_t = ttt::update_scan_segments(p->d, p->d, p->kk, Cw);
  p->DFm = std::max(2 * p->f * p->d, p->d * p->d);
  p->npart = ttt::conv_bwd_partials(p->B * p->n);
  if (p->B * p->n == 0) return TTT_OK;        // nothing but zero weight gradients
  size_t off = 0;
  auto take = [&](size_t* o, size_t bytes) {
    *o = off;
    off += align_up(bytes);
  };
  const size_t BN = (size_t)p->B * p->n, e = p->esz, DFm = (size_t)p->DFm, B = (size_t)p->B;
  const int Smax = std::max(p->S_gu, p->S_t);
  take(&p->off_Z, BN * p->f * e);
  take(&p->off_Y, BN * p->d * e);
  take(&p->off_WtT, (size_t)p->d * p->d * e);
  if (mode == TTT_MODE_MSE) take(&p->off_V, BN * p->d * e);      // V^ itself (the dot core keeps eta V^)
  take(&p->off_dZ, BN * p->f * e);
  take(&p->off_dV, BN * p->d * e);
  take(&p->off_G, BN * 2 * p->f * e);
  take(&p->off_dY, BN * p->d * e);
  take(&p->off_wWc, B * p->kk * DFm * e);
  if (Smax > 1) {
    take(&p->off_wWp, B * (p->kk - p->kk / Smax) * DFm * e);
    take(&p->off_wTot, B * (Smax - 1) * DFm * 4);
  }
  take(&p->off_wWf, B * DFm * 4);
  take(&p->off_wzero, DFm * e);
  take(&p->off_part, (size_t)p->npart * p->d * p->K * 4);
  take(&p->off_core, mode == TTT_MODE_MSE ? p->mcore.total : p->core.total);
  p->total = off;
  return TTT_OK;
}

// Sum over the rows and tokens of Q^T P (Q [B, n, dq], P [B, n, fp], row-major):
// the fused update-scan from a zero state, its per-row totals in wWf [B, dq, fp].
template <typename T>
int token_contraction(const LayerBwdPlan& L, const T* P, const T* Q, int dq, int fp, int S, char* ws, hipStream_t s) {
  const int B = (int)L.B, n = (int)L.n, Cw = (int)(L.n / L.kk);
  return dev(ttt::launch_chunk_update_scan<T>(P, Q, (const T*)(ws + L.off_wzero), (T*)(ws + L.off_wWc),
                                              (float*)(ws + L.off_wWf), (T*)(ws + L.off_wWp),
                                              (float*)(ws + L.off_wTot), B, n, dq, fp, Cw, S, nullptr, nullptr, s,
                                              ttt::kScanRowMajor));
}

template <typename T>
int layer_backward(const LayerBwdPlan& L, float eta, const void* Hv, const void* X0v, const void* Wgv,
                   const void* Wuv, const void* W0, const void* Wtv, const void* cwv, const void* dO,
                   const void* Wsaved, void* dHv, void* dX0v, float* dWg, float* dWu, float* dW0, float* dWt,
                   float* dcw, char* ws, hipStream_t s) {
  const int B = (int)L.B, n = (int)L.n, d = (int)L.d, f = (int)L.f, C = (int)L.C, K = (int)L.K;
  const int64_t rows = L.B * L.n, fd = (int64_t)f * d;
  const bool mse = L.mode == TTT_MODE_MSE;
  if (rows == 0) {
    int st = dev(ttt::launch_zero<float>(dWg, fd, s));
    if (st == TTT_OK) st = dev(ttt::launch_zero<float>(dWu, fd, s));
    if (st == TTT_OK) st = dev(ttt::launch_zero<float>(dW0, fd, s));
    if (st == TTT_OK) st = dev(ttt::launch_zero<float>(dWt, (int64_t)d * d, s));
    if (st == TTT_OK) st = dev(ttt::launch_zero<float>(dcw, (int64_t)d * K, s));
    const float* Wi = mse ? L.mcore.Winit : L.core.Winit;
    if (st == TTT_OK && Wi != nullptr)
      st = dev(ttt::launch_zero<float>(mse ? L.mcore.dWi : L.core.dWi, L.B * (int64_t)d * f, s));
    if (st == TTT_OK && L.dhalo != nullptr) st = dev(ttt::launch_zero<T>((T*)L.dhalo, L.B * (K - 1) * (int64_t)d, s));
    return st;
  }
  const T* H = (const T*)Hv;
  const T* Wg = (const T*)Wgv;
  const T* Wu = (const T*)Wuv;
  const T* Wt = (const T*)Wtv;
  T* Z = (T*)(ws + L.off_Z);
  T* Y = (T*)(ws + L.off_Y);
  T* WtT = (T*)(ws + L.off_WtT);
  T* dZ = (T*)(ws + L.off_dZ);
  T* dV = (T*)(ws + L.off_dV);
  T* G = (T*)(ws + L.off_G);
  T* dY = (T*)(ws + L.off_dY);
  float* wWf = (float*)(ws + L.off_wWf);
  float* part = (float*)(ws + L.off_part);
  char* cws = ws + L.off_core;
  const uint8_t* docs = mse ? L.mcore.docs : L.core.docs;
  // the target as the chunk loop's backward takes it: eta V^ in the dot core's own buffer, V^ for MSE
  T* Vs = mse ? (T*)(ws + L.off_V) : (T*)(cws + L.core.off_Vs);
  // the forward's activations: Z (eq. (2)), Y = Conv1D(X0), V^ = Y W_target (eq. (5))
  int st = dev(ttt::launch_zero<T>((T*)(ws + L.off_wzero), L.DFm, s));
  if (st == TTT_OK) st = dev(ttt::launch_produce_z<T>(H, Wg, Wu, Z, nullptr, rows, n, d, f, s));
  if (st == TTT_OK)
    st = dev(ttt::launch_conv<T>((const T*)X0v, (const T*)cwv, Y, rows, n, d, K, docs, C, L.conv_fwd,
                                 (const T*)L.halo, s));
  if (st == TTT_OK) st = dev(ttt::launch_transpose<T>(Wt, WtT, 1, d, d, 1.0f, 0, s));
  if (st == TTT_OK) st = dev(ttt::launch_apply<T>(Y, WtT, 0, 0, Vs, B, n, d, d, C, mse ? 1.0f : eta, s, true));
  // the chunk loop: dZ, dV^ and dW_down0
  if (st == TTT_OK)
    st = mse ? mse_backward<T>(L.mcore, eta, Z, Vs, W0, dO, Wsaved, dZ, dV, dW0, cws, s)
             : core_backward<T>(L.core, eta, Z, nullptr, W0, dO, Wsaved, dZ, dV, dW0, cws, s, true);
  // the producer: [dA | dU], then [dW_gate; dW_up] = sum G^T H and dH = dA W_gate + dU W_up
  if (st == TTT_OK) st = dev(ttt::launch_produce_z_bwd<T>(H, Wg, Wu, dZ, G, rows, n, d, f, s));
  if (st == TTT_OK) st = token_contraction<T>(L, H, G, 2 * f, d, L.S_gu, ws, s);
  if (st == TTT_OK) st = dev(ttt::launch_sum_rows(wWf, dWg, B, fd, s, 2 * fd));
  if (st == TTT_OK) st = dev(ttt::launch_sum_rows(wWf + fd, dWu, B, fd, s, 2 * fd));
  if (st == TTT_OK)
    st = dev(ttt::launch_dz<T>(G + f, G, Wu, 0, 0, Wg, 0, 0, (T*)dHv, B, n, f, d, C, s, 2 * f));
  // the target: dW_target = sum Y^T dV^, dY = dV^ W_target^T, then the convolution's taps and input
  if (st == TTT_OK) st = token_contraction<T>(L, dV, Y, d, d, L.S_t, ws, s);
  if (st == TTT_OK) st = dev(ttt::launch_sum_rows(wWf, dWt, B, (int64_t)d * d, s));
  if (st == TTT_OK) st = dev(ttt::launch_apply<T>(dV, Wt, 0, 0, dY, B, n, d, d, C, 1.0f, s, true));
  if (st == TTT_OK)
    st = dev(ttt::launch_conv_bwd<T>((const T*)X0v, (const T*)cwv, dY, (T*)dX0v, part, rows, n, d, K, s, docs, C,
                                     L.conv_fwd, (const T*)L.halo, (T*)L.dhalo));
  if (st == TTT_OK) st = dev(ttt::launch_sum_rows(part, dcw, (int)L.npart, (int64_t)d * K, s));
  return st;
}

// Plan and argument checks of the whole layer's call (every pointer the shape
// needs present and 16-byte aligned, eta finite).
int layer_plan(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* H, const void* X0,
               const void* W_gate, const void* W_up, const void* W_down0, const void* W_target, const void* conv_w,
               const void* O, const float* W_final, Plan* p) {
  int st = make_plan(shape, dtype, mode, true, p);
  if (st != TTT_OK) return st;
  if (!finite(eta)) return TTT_ERR_ARG;
  if (p->B > 0) {
    if (!ok_ptr(W_down0) || !ok_ptr(W_final)) return TTT_ERR_ARG;
    if (p->n > 0 && (!ok_ptr(H) || !ok_ptr(X0) || !ok_ptr(W_gate) || !ok_ptr(W_up) || !ok_ptr(W_target) ||
                     !ok_ptr(conv_w) || !ok_ptr(O)))
      return TTT_ERR_ARG;
  }
  return TTT_OK;
}

// ------------------------------------------------------------------ static scratch (no allocation)

// The scratch of ttt_chunk_apply_update_noalloc: a device array in the
// library's code object, so each device that loads the library holds its own
// copy from the first use until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device copy: kernels and copies take
// the address hipGetSymbolAddress gives for the device, kept per device below.
static __device__ __align__(256) char scratch[TTT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<char*> g_scratch_addr[kMaxDevices];

// Makes dev the current device for the guard's lifetime.
struct DeviceGuard {
  int prev = -1;
  hipError_t enter(int dev) {
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    else prev = -1;
    return e;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

// The device address of `scratch` on the device of stream s, looked up on the
// first call for that device (with the device current) and kept.
int static_scratch(hipStream_t s, char** out) {
  int devid = -1;
  if (hipStreamGetDevice(s, &devid) != hipSuccess || devid < 0 || devid >= kMaxDevices) return TTT_ERR_DEVICE;
  char* p = g_scratch_addr[devid].load(std::memory_order_acquire);
  if (p == nullptr) {
    DeviceGuard guard;
    if (guard.enter(devid) != hipSuccess) return TTT_ERR_DEVICE;
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return TTT_ERR_DEVICE;
    p = (char*)addr;
    g_scratch_addr[devid].store(p, std::memory_order_release);   // every thread finds the same address
  }
  *out = p;
  return TTT_OK;
}

int core_backward_call(int mode, const ttt_inplace_shape* shape, int dtype, float eta, const void* Z, const void* Vhat,
                       const void* W_down0, const void* dO, const ttt_backward_options* o, void* dZ, void* dVhat,
                       float* dW_down0, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace

extern "C" {

const char* ttt_status_string(int status) {
  switch (status) {
    case TTT_OK: return "TTT_OK";
    case TTT_ERR_ARG: return "TTT_ERR_ARG: null or misaligned pointer, unknown mode/order, or non-finite eta";
    case TTT_ERR_SHAPE: return "TTT_ERR_SHAPE: negative or zero size, or seq_len not a multiple of chunk";
    case TTT_ERR_DTYPE: return "TTT_ERR_DTYPE: dtype must be TTT_F32 or TTT_BF16";
    case TTT_ERR_WORKSPACE: return "TTT_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case TTT_ERR_DEVICE: return "TTT_ERR_DEVICE: the HIP runtime rejected a launch";
    case TTT_ERR_UNSUPPORTED: return "TTT_ERR_UNSUPPORTED: sizes outside what this build handles";
    case TTT_ERR_SCRATCH_LIMIT:
      return "TTT_ERR_SCRATCH_LIMIT: the call needs more scratch than the static buffer of the allocation-free "
             "entry point holds (TTT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int ttt_inplace_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int mode, int with_producers,
                                size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  Plan p;
  int st = make_plan(shape, dtype, mode, with_producers != 0, &p);
  if (st != TTT_OK) return st;
  *bytes = p.total;
  return TTT_OK;
}

int ttt_chunk_apply_update(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* H,
                           const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
                           const void* W_target, const void* conv_w, void* O, float* W_final, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Plan p;
  int st = layer_plan(shape, dtype, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, &p);
  if (st != TTT_OK) return st;
  if ((st = check_ws(p, workspace, workspace_bytes)) != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (dtype == TTT_BF16)
    return layer<bf16>(p, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, ws, s);
  return layer<float>(p, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, ws, s);
}

int ttt_chunk_apply_update_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* H,
                              const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
                              const void* W_target, const void* conv_w, const ttt_layer_options* options, void* O,
                              float* W_final, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = layer_plan(shape, dtype, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, &p);
  if (st != TTT_OK) return st;
  if ((st = check_ws(p, workspace, workspace_bytes)) != TTT_OK) return st;
  if ((st = apply_options(p, mode, options, true)) != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (dtype == TTT_BF16)
    return layer<bf16>(p, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, ws, s);
  return layer<float>(p, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, ws, s);
}

int ttt_chunk_apply_update_noalloc(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* H,
                                   const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
                                   const void* W_target, const void* conv_w, void* O, float* W_final, void* stream) {
  Plan p;
  int st = layer_plan(shape, dtype, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, &p);
  if (st != TTT_OK) return st;
  if (p.total > (size_t)TTT_NOALLOC_SCRATCH_BYTES) return TTT_ERR_SCRATCH_LIMIT;
  hipStream_t s = (hipStream_t)stream;
  char* ws = nullptr;
  if (p.total > 0 && (st = static_scratch(s, &ws)) != TTT_OK) return st;
  if (dtype == TTT_BF16)
    return layer<bf16>(p, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, ws, s);
  return layer<float>(p, mode, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, O, W_final, ws, s);
}

int ttt_core_apply_update(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* Z,
                          const void* Vhat, const void* W_down0, void* O, float* W_final, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return ttt_core_apply_update_ex(shape, dtype, mode, eta, Z, Vhat, W_down0, nullptr, O, W_final, workspace,
                                  workspace_bytes, stream);
}

int ttt_core_apply_update_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* Z,
                             const void* Vhat, const void* W_down0, const ttt_layer_options* options, void* O,
                             float* W_final, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, dtype, mode, false, &p);
  if (st != TTT_OK) return st;
  if (!finite(eta)) return TTT_ERR_ARG;
  if (p.B > 0) {
    if (!ok_ptr(W_down0) || !ok_ptr(W_final)) return TTT_ERR_ARG;
    if (p.n > 0 && (!ok_ptr(Z) || !ok_ptr(Vhat) || !ok_ptr(O))) return TTT_ERR_ARG;
  }
  if ((st = check_ws(p, workspace, workspace_bytes)) != TTT_OK) return st;
  if ((st = apply_options(p, mode, options, false)) != TTT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == TTT_BF16) return core<bf16>(p, mode, eta, Z, Vhat, W_down0, O, W_final, (char*)workspace, s);
  return core<float>(p, mode, eta, Z, Vhat, W_down0, O, W_final, (char*)workspace, s);
}

int ttt_core_backward_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states, size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  BwdPlan p;
  int st = make_bwd_plan(shape, dtype, saved_states != 0, &p, true);
  if (st != TTT_OK) return st;
  *bytes = p.total;
  return TTT_OK;
}

int ttt_core_backward(const ttt_inplace_shape* shape, int dtype, float eta, const void* Z, const void* Vhat,
                      const void* W_down0, const void* dO, const void* W_states, const unsigned char* doc_starts,
                      void* dZ, void* dVhat, float* dW_down0, void* workspace, size_t workspace_bytes, void* stream) {
  const ttt_backward_options o{W_states, doc_starts, nullptr, 0};
  return core_backward_call(TTT_MODE_DOT, shape, dtype, eta, Z, Vhat, W_down0, dO, &o, dZ, dVhat, dW_down0, workspace,
                            workspace_bytes, stream);
}

int ttt_core_backward_mse_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states,
                                          size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  MsePlan p;
  int st = make_mse_plan(shape, dtype, &p, saved_states != 0);
  if (st != TTT_OK) return st;
  *bytes = p.total;
  return TTT_OK;
}

int ttt_core_backward_mse(const ttt_inplace_shape* shape, int dtype, float eta, const void* Z, const void* Vhat,
                          const void* W_down0, const void* dO, const void* W_states, const unsigned char* doc_starts,
                          void* dZ, void* dVhat, float* dW_down0, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const ttt_backward_options o{W_states, doc_starts, nullptr, 0};
  return core_backward_call(TTT_MODE_MSE, shape, dtype, eta, Z, Vhat, W_down0, dO, &o, dZ, dVhat, dW_down0, workspace,
                            workspace_bytes, stream);
}

int ttt_layer_backward_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states, size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  LayerBwdPlan p;
  int st = make_layer_bwd_plan(shape, dtype, saved_states != 0, &p);
  if (st != TTT_OK) return st;
  *bytes = p.total;
  return TTT_OK;
}

int ttt_layer_backward_mse_workspace_bytes(const ttt_inplace_shape* shape, int dtype, int saved_states,
                                           size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  LayerBwdPlan p;
  int st = make_layer_bwd_plan(shape, dtype, saved_states != 0, &p, TTT_MODE_MSE);
  if (st != TTT_OK) return st;
  *bytes = p.total;
  return TTT_OK;
}

}  // extern "C"

namespace {

// The resumed rows' fields of backward options: each gradient goes with its
// input (both present and 16-byte aligned, or both null; with no batch rows
// nothing is read); halo: whether x0_halo / dx0_halo are read at all.
bool resume_args_ok(const ttt_backward_options* o, bool rows, bool halo) {
  if ((o->W_init == nullptr) != (o->dW_init == nullptr)) return false;
  if (rows && o->W_init != nullptr && (!ok_ptr(o->W_init) || !ok_ptr(o->dW_init))) return false;
  if (!halo) return true;
  if ((o->x0_halo == nullptr) != (o->dx0_halo == nullptr)) return false;
  return o->x0_halo == nullptr || (ok_ptr(o->x0_halo) && ok_ptr(o->dx0_halo));
}

// The whole layer's backward for either objective (the entry points below).
int layer_backward_call(int mode, const ttt_inplace_shape* shape, int dtype, float eta, const void* H, const void* X0,
                        const void* W_gate, const void* W_up, const void* W_down0, const void* W_target,
                        const void* conv_w, const void* dO, const ttt_backward_options* o, void* dH, void* dX0,
                        float* dW_gate, float* dW_up, float* dW_down0, float* dW_target, float* dconv_w,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const ttt_backward_options none{};
  if (o == nullptr) o = &none;
  if (mode == TTT_MODE_DOT_SCAN) mode = TTT_MODE_DOT;
  if ((mode != TTT_MODE_DOT && mode != TTT_MODE_MSE) || (o->conv_forward != 0 && o->conv_forward != 1))
    return TTT_ERR_ARG;
  LayerBwdPlan p;
  int st = make_layer_bwd_plan(shape, dtype, o->W_states != nullptr, &p, mode);
  if (st != TTT_OK) return st;
  p.core.docs = p.mcore.docs = o->doc_starts;
  p.core.umask = p.mcore.umask = o->update_mask;
  p.core.Winit = p.mcore.Winit = o->W_init;
  p.core.dWi = p.mcore.dWi = o->dW_init;
  p.conv_fwd = o->conv_forward == 1;
  p.halo = p.K > 1 ? o->x0_halo : nullptr;
  p.dhalo = p.K > 1 ? o->dx0_halo : nullptr;
  if (!finite(eta) || !resume_args_ok(o, p.B > 0, p.B > 0 && p.K > 1)) return TTT_ERR_ARG;
  if (!ok_ptr(dW_gate) || !ok_ptr(dW_up) || !ok_ptr(dW_down0) || !ok_ptr(dW_target) || !ok_ptr(dconv_w) ||
      (o->W_states != nullptr && !aligned16(o->W_states)))
    return TTT_ERR_ARG;
  if (p.B * p.n > 0 && (!ok_ptr(H) || !ok_ptr(X0) || !ok_ptr(W_gate) || !ok_ptr(W_up) || !ok_ptr(W_down0) ||
                        !ok_ptr(W_target) || !ok_ptr(conv_w) || !ok_ptr(dO) || !ok_ptr(dH) || !ok_ptr(dX0)))
    return TTT_ERR_ARG;
  if (p.total > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < p.total))
    return TTT_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (dtype == TTT_BF16)
    return layer_backward<bf16>(p, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, o->W_states, dH, dX0,
                                dW_gate, dW_up, dW_down0, dW_target, dconv_w, ws, s);
  return layer_backward<float>(p, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, o->W_states, dH, dX0,
                               dW_gate, dW_up, dW_down0, dW_target, dconv_w, ws, s);
}

// The chunk loop's backward for either objective (the entry points below).
int core_backward_call(int mode, const ttt_inplace_shape* shape, int dtype, float eta, const void* Z, const void* Vhat,
                       const void* W_down0, const void* dO, const ttt_backward_options* o, void* dZ, void* dVhat,
                       float* dW_down0, void* workspace, size_t workspace_bytes, void* stream) {
  const ttt_backward_options none{};
  if (o == nullptr) o = &none;
  if (mode == TTT_MODE_DOT_SCAN) mode = TTT_MODE_DOT;
  if (mode != TTT_MODE_DOT && mode != TTT_MODE_MSE) return TTT_ERR_ARG;
  const void* Ws = o->W_states;
  size_t total;
  BwdPlan p;
  MsePlan q;
  int st = mode == TTT_MODE_MSE ? make_mse_plan(shape, dtype, &q, Ws != nullptr)
                                : make_bwd_plan(shape, dtype, Ws != nullptr, &p, true);
  if (st != TTT_OK) return st;
  const int64_t BN = mode == TTT_MODE_MSE ? q.B * q.n : p.B * p.n;
  total = mode == TTT_MODE_MSE ? q.total : p.total;
  p.docs = q.docs = o->doc_starts;
  p.umask = q.umask = o->update_mask;
  p.Winit = q.Winit = o->W_init;
  p.dWi = q.dWi = o->dW_init;
  if (!finite(eta) || !ok_ptr(dW_down0) || (Ws != nullptr && !aligned16(Ws)) ||
      !resume_args_ok(o, (mode == TTT_MODE_MSE ? q.B : p.B) > 0, false))
    return TTT_ERR_ARG;
  if (BN > 0 && (!ok_ptr(Z) || !ok_ptr(Vhat) || !ok_ptr(W_down0) || !ok_ptr(dO) || !ok_ptr(dZ) || !ok_ptr(dVhat)))
    return TTT_ERR_ARG;
  if (total > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < total))
    return TTT_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (mode == TTT_MODE_MSE)
    return dtype == TTT_BF16 ? mse_backward<bf16>(q, eta, Z, Vhat, W_down0, dO, Ws, dZ, dVhat, dW_down0, ws, s)
                             : mse_backward<float>(q, eta, Z, Vhat, W_down0, dO, Ws, dZ, dVhat, dW_down0, ws, s);
  return dtype == TTT_BF16 ? core_backward<bf16>(p, eta, Z, Vhat, W_down0, dO, Ws, dZ, dVhat, dW_down0, ws, s)
                           : core_backward<float>(p, eta, Z, Vhat, W_down0, dO, Ws, dZ, dVhat, dW_down0, ws, s);
}

}  // namespace

extern "C" {

int ttt_layer_backward(const ttt_inplace_shape* shape, int dtype, float eta, const void* H, const void* X0,
                       const void* W_gate, const void* W_up, const void* W_down0, const void* W_target,
                       const void* conv_w, const void* dO, const void* W_states, const unsigned char* doc_starts,
                       void* dH, void* dX0, float* dW_gate, float* dW_up, float* dW_down0, float* dW_target,
                       float* dconv_w, void* workspace, size_t workspace_bytes, void* stream) {
  const ttt_backward_options o{W_states, doc_starts, nullptr, 0};
  return layer_backward_call(TTT_MODE_DOT, shape, dtype, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, &o,
                             dH, dX0, dW_gate, dW_up, dW_down0, dW_target, dconv_w, workspace, workspace_bytes, stream);
}

int ttt_layer_backward_mse(const ttt_inplace_shape* shape, int dtype, float eta, const void* H, const void* X0,
                           const void* W_gate, const void* W_up, const void* W_down0, const void* W_target,
                           const void* conv_w, const void* dO, const void* W_states, const unsigned char* doc_starts,
                           void* dH, void* dX0, float* dW_gate, float* dW_up, float* dW_down0, float* dW_target,
                           float* dconv_w, void* workspace, size_t workspace_bytes, void* stream) {
  const ttt_backward_options o{W_states, doc_starts, nullptr, 0};
  return layer_backward_call(TTT_MODE_MSE, shape, dtype, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, &o,
                             dH, dX0, dW_gate, dW_up, dW_down0, dW_target, dconv_w, workspace, workspace_bytes, stream);
}

int ttt_layer_backward_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* H,
                          const void* X0, const void* W_gate, const void* W_up, const void* W_down0,
                          const void* W_target, const void* conv_w, const void* dO,
                          const ttt_backward_options* options, void* dH, void* dX0, float* dW_gate, float* dW_up,
                          float* dW_down0, float* dW_target, float* dconv_w, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return layer_backward_call(mode, shape, dtype, eta, H, X0, W_gate, W_up, W_down0, W_target, conv_w, dO, options, dH,
                             dX0, dW_gate, dW_up, dW_down0, dW_target, dconv_w, workspace, workspace_bytes, stream);
}

int ttt_core_backward_ex(const ttt_inplace_shape* shape, int dtype, int mode, float eta, const void* Z,
                         const void* Vhat, const void* W_down0, const void* dO, const ttt_backward_options* options,
                         void* dZ, void* dVhat, float* dW_down0, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return core_backward_call(mode, shape, dtype, eta, Z, Vhat, W_down0, dO, options, dZ, dVhat, dW_down0, workspace,
                            workspace_bytes, stream);
}

int ttt_produce_z(const ttt_inplace_shape* shape, int dtype, const void* H, const void* W_gate, const void* W_up,
                  void* Z, void* Zt, void* stream) {
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  const int64_t rows = shape->batch * shape->seq_len;
  if (rows == 0) return TTT_OK;
  if (!ok_ptr(H) || !ok_ptr(W_gate) || !ok_ptr(W_up) || !ok_ptr(Zt) || (Z != nullptr && !aligned16(Z)))
    return TTT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int n = (int)shape->seq_len, d = (int)shape->d_model, f = (int)shape->d_ff;
  if (dtype == TTT_BF16)
    return dev(ttt::launch_produce_z<bf16>((const bf16*)H, (const bf16*)W_gate, (const bf16*)W_up, (bf16*)Z,
                                           (bf16*)Zt, rows, n, d, f, s));
  return dev(ttt::launch_produce_z<float>((const float*)H, (const float*)W_gate, (const float*)W_up, (float*)Z,
                                          (float*)Zt, rows, n, d, f, s));
}

int ttt_vhat_workspace_bytes(const ttt_inplace_shape* shape, int dtype, size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  const size_t e = dtype == TTT_BF16 ? 2 : 4;
  *bytes = align_up((size_t)shape->batch * shape->seq_len * shape->d_model * e) +
           align_up((size_t)shape->d_model * shape->d_model * e);
  return TTT_OK;
}

int ttt_produce_vhat(const ttt_inplace_shape* shape, int dtype, float scale, const void* X0, const void* conv_w,
                     const void* W_target, void* Vt, void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  int st = ttt_vhat_workspace_bytes(shape, dtype, &need);
  if (st != TTT_OK) return st;
  if (!finite(scale)) return TTT_ERR_ARG;
  const int64_t rows = shape->batch * shape->seq_len;
  if (rows == 0) return TTT_OK;
  if (!ok_ptr(X0) || !ok_ptr(conv_w) || !ok_ptr(W_target) || !ok_ptr(Vt)) return TTT_ERR_ARG;
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return TTT_ERR_WORKSPACE;
  Plan p{};
  p.B = shape->batch;
  p.n = shape->seq_len;
  p.d = shape->d_model;
  p.K = shape->conv_k;
  const size_t e = dtype == TTT_BF16 ? 2 : 4;
  p.off_Y = 0;
  p.off_WtT = align_up((size_t)rows * p.d * e);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int n = (int)p.n, d = (int)p.d, K = (int)p.K;
  if (dtype == TTT_BF16) {
    st = dev(ttt::launch_conv<bf16>((const bf16*)X0, (const bf16*)conv_w, (bf16*)(ws + p.off_Y), rows, n, d, K, nullptr,
                                    (int)p.C, false, nullptr, s));
    if (st == TTT_OK)
      st = dev(ttt::launch_transpose<bf16>((const bf16*)W_target, (bf16*)(ws + p.off_WtT), 1, d, d, 1.0f, 0, s));
    if (st == TTT_OK)
      st = dev(ttt::launch_produce_vhat<bf16>((const bf16*)(ws + p.off_Y), (const bf16*)(ws + p.off_WtT), (bf16*)Vt,
                                              rows, n, d, scale, s));
    return st;
  }
  st = dev(ttt::launch_conv<float>((const float*)X0, (const float*)conv_w, (float*)(ws + p.off_Y), rows, n, d, K,
                                   nullptr, (int)p.C, false, nullptr, s));
  if (st == TTT_OK)
    st = dev(ttt::launch_transpose<float>((const float*)W_target, (float*)(ws + p.off_WtT), 1, d, d, 1.0f, 0, s));
  if (st == TTT_OK)
    st = dev(ttt::launch_produce_vhat<float>((const float*)(ws + p.off_Y), (const float*)(ws + p.off_WtT),
                                             (float*)Vt, rows, n, d, scale, s));
  return st;
}

int ttt_chunk_delta(const ttt_inplace_shape* shape, int dtype, const void* Zt, const void* Vt, float* dW,
                    void* stream) {
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  if (shape->batch * shape->seq_len == 0) return TTT_OK;
  if (!ok_ptr(Zt) || !ok_ptr(Vt) || !ok_ptr(dW)) return TTT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int B = (int)shape->batch, n = (int)shape->seq_len, d = (int)shape->d_model, f = (int)shape->d_ff,
            C = (int)shape->chunk;
  if (dtype == TTT_BF16)
    return dev(ttt::launch_chunk_delta<bf16>((const bf16*)Zt, (const bf16*)Vt, dW, B, n, d, f, C, s));
  return dev(ttt::launch_chunk_delta<float>((const float*)Zt, (const float*)Vt, dW, B, n, d, f, C, s));
}

int ttt_chunk_scan(const ttt_inplace_shape* shape, int dtype, float eta, const void* W_down0, const float* dW,
                   void* Wc, float* W_final, void* stream) {
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  if (!finite(eta)) return TTT_ERR_ARG;
  if (shape->batch == 0) return TTT_OK;
  const int k = (int)(shape->seq_len / shape->chunk);
  if (!ok_ptr(W_down0) || !ok_ptr(W_final)) return TTT_ERR_ARG;
  if (k > 0 && (!ok_ptr(dW) || !ok_ptr(Wc))) return TTT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int64_t df = shape->d_model * shape->d_ff;
  if (dtype == TTT_BF16)
    return dev(ttt::launch_chunk_scan<bf16>(dW, (const bf16*)W_down0, (bf16*)Wc, W_final, (int)shape->batch, k, df,
                                            eta, nullptr, nullptr, s));
  return dev(ttt::launch_chunk_scan<float>(dW, (const float*)W_down0, (float*)Wc, W_final, (int)shape->batch, k, df,
                                           eta, nullptr, nullptr, s));
}

static size_t update_scan_ws(const ttt_inplace_shape* s, int dtype) {
  const int64_t k = s->seq_len / s->chunk;
  const int S = ttt::update_scan_segments(s->d_model, s->d_ff, k, s->chunk);
  if (S == 1) return 0;
  const size_t DF = (size_t)s->d_model * s->d_ff;
  const size_t esz = dtype == TTT_BF16 ? 2 : 4;
  return align_up((size_t)s->batch * (k - k / S) * DF * esz) + align_up((size_t)s->batch * (S - 1) * DF * 4);
}

int ttt_update_scan_workspace_bytes(const ttt_inplace_shape* shape, int dtype, size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  if (shape->chunk % kstep(dtype) != 0) return TTT_ERR_UNSUPPORTED;
  *bytes = update_scan_ws(shape, dtype);
  return TTT_OK;
}

int ttt_chunk_update_scan(const ttt_inplace_shape* shape, int dtype, const void* W_down0, const void* Zt,
                          const void* Vt, void* Wc, float* W_final, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  if (shape->chunk % kstep(dtype) != 0) return TTT_ERR_UNSUPPORTED;
  if (shape->batch == 0) return TTT_OK;
  if (!ok_ptr(W_down0) || !ok_ptr(W_final)) return TTT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int B = (int)shape->batch, n = (int)shape->seq_len, d = (int)shape->d_model, f = (int)shape->d_ff,
            C = (int)shape->chunk;
  const int64_t df = (int64_t)d * f;
  if (n == 0) {
    if (dtype == TTT_BF16)
      return dev(ttt::launch_chunk_scan<bf16>(nullptr, (const bf16*)W_down0, nullptr, W_final, B, 0, df, 0.f, nullptr,
                                                nullptr, s));
    return dev(ttt::launch_chunk_scan<float>(nullptr, (const float*)W_down0, nullptr, W_final, B, 0, df, 0.f,
                                                 nullptr, nullptr, s));
  }
  if (!ok_ptr(Zt) || !ok_ptr(Vt) || !ok_ptr(Wc)) return TTT_ERR_ARG;
  const size_t need = update_scan_ws(shape, dtype);
  if (workspace_bytes < need || (need > 0 && !ok_ptr(workspace))) return TTT_ERR_WORKSPACE;
  const int k = n / C, S = ttt::update_scan_segments(d, f, k, C);
  char* ws = (char*)workspace;
  const size_t esz = dtype == TTT_BF16 ? 2 : 4;
  void* Wp = S > 1 ? (void*)ws : nullptr;
  float* Tot = S > 1 ? (float*)(ws + align_up((size_t)B * (k - k / S) * df * esz)) : nullptr;
  if (dtype == TTT_BF16)
    return dev(ttt::launch_chunk_update_scan<bf16>((const bf16*)Zt, (const bf16*)Vt, (const bf16*)W_down0, (bf16*)Wc,
                                                   W_final, (bf16*)Wp, Tot, B, n, d, f, C, S, nullptr,
                                                   nullptr, s));
  return dev(ttt::launch_chunk_update_scan<float>((const float*)Zt, (const float*)Vt, (const float*)W_down0,
                                                  (float*)Wc, W_final, (float*)Wp, Tot, B, n, d, f, C, S, nullptr,
                                                  nullptr, s));
}

int ttt_chunk_apply(const ttt_inplace_shape* shape, int dtype, const void* Zt, const void* Wc, void* O, void* stream) {
  int st = check_inplace_shape(shape, dtype);
  if (st != TTT_OK) return st;
  if (shape->batch * shape->seq_len == 0) return TTT_OK;
  if (!ok_ptr(Zt) || !ok_ptr(Wc) || !ok_ptr(O)) return TTT_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const int B = (int)shape->batch, n = (int)shape->seq_len, d = (int)shape->d_model, f = (int)shape->d_ff,
            C = (int)shape->chunk;
  const int64_t df = (int64_t)d * f, k = n / C;
  if (dtype == TTT_BF16)
    return dev(
        ttt::launch_apply<bf16>((const bf16*)Zt, (const bf16*)Wc, k * df, df, (bf16*)O, B, n, d, f, C, 1.0f, s));
  return dev(
      ttt::launch_apply<float>((const float*)Zt, (const float*)Wc, k * df, df, (float*)O, B, n, d, f, C, 1.0f, s));
}

// ------------------------------------------------------------------ LaCT

static int check_lact(const ttt_lact_shape* s, int dtype) {
  if (s == nullptr) return TTT_ERR_ARG;
  if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_ERR_DTYPE;
  if (s->batch < 0 || s->heads <= 0 || s->seq_len < 0 || s->head_dim <= 0 || s->hidden <= 0 || s->chunk <= 0)
    return TTT_ERR_SHAPE;
  if (s->seq_len % s->chunk != 0) return TTT_ERR_SHAPE;
  if (s->head_dim % 8 || s->hidden % 8 || s->chunk % 8) return TTT_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 30;
  if (s->head_dim > 8192 || s->hidden > 65536 || s->seq_len > lim || s->batch * s->heads > 65536 ||
      s->batch * s->heads * s->seq_len > lim)
    return TTT_ERR_UNSUPPORTED;
  return TTT_OK;
}

int ttt_lact_workspace_bytes(const ttt_lact_shape* shape, int dtype, size_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_ARG;
  int st = check_lact(shape, dtype);
  if (st != TTT_OK) return st;
  const int B = (int)shape->batch, H = (int)shape->heads, n = (int)shape->seq_len, dh = (int)shape->head_dim,
            m = (int)shape->hidden, C = (int)shape->chunk;
  *bytes = dtype == TTT_BF16 ? ttt::lact_workspace_bytes<bf16>(B, H, n, dh, m, C)
                             : ttt::lact_workspace_bytes<float>(B, H, n, dh, m, C);
  return TTT_OK;
}

int ttt_lact_swiglu(const ttt_lact_shape* shape, int dtype, int order, float eta, const void* q, const void* k,
                    const void* v, const void* W1, const void* W3, const void* W2, void* O, float* W1_f, float* W3_f,
                    float* W2_f, void* workspace, size_t workspace_bytes, void* stream) {
  ttt_lact_options opt{};
  opt.order = order;
  return ttt_lact_swiglu_ex(shape, dtype, eta, q, k, v, W1, W3, W2, &opt, O, W1_f, W3_f, W2_f, workspace,
                            workspace_bytes, stream);
}

int ttt_lact_backward_workspace_bytes(const ttt_lact_shape* shape, int dtype, size_t* bytes) {
  return ttt_lact_backward_workspace_bytes_ex(shape, dtype, 0, bytes);
}

int ttt_lact_backward_workspace_bytes_ex(const ttt_lact_shape* shape, int dtype, int saved_states, size_t* bytes) {
  if (bytes == nullptr || (saved_states != 0 && saved_states != 1)) return TTT_ERR_ARG;
  int st = check_lact(shape, dtype);
  if (st != TTT_OK) return st;
  const int B = (int)shape->batch, H = (int)shape->heads, n = (int)shape->seq_len, dh = (int)shape->head_dim,
            m = (int)shape->hidden, C = (int)shape->chunk;
  *bytes = dtype == TTT_BF16 ? ttt::lact_bwd_workspace_bytes<bf16>(B, H, n, dh, m, C, saved_states != 0)
                             : ttt::lact_bwd_workspace_bytes<float>(B, H, n, dh, m, C, saved_states != 0);
  return TTT_OK;
}

int ttt_lact_swiglu_backward(const ttt_lact_shape* shape, int dtype, int order, float eta, const void* q,
                             const void* k, const void* v, const void* W1, const void* W3, const void* W2,
                             const void* dO, void* dq, void* dk, void* dv, float* dW1, float* dW3, float* dW2,
                             void* workspace, size_t workspace_bytes, void* stream) {
  ttt_lact_options opt{};
  opt.order = order;
  return ttt_lact_swiglu_backward_ex(shape, dtype, eta, q, k, v, W1, W3, W2, dO, &opt, dq, dk, dv, dW1, dW3, dW2,
                                     workspace, workspace_bytes, stream);
}

int ttt_lact_swiglu_backward_ex(const ttt_lact_shape* shape, int dtype, float eta, const void* q, const void* k,
                                const void* v, const void* W1, const void* W3, const void* W2, const void* dO,
                                const ttt_lact_options* options, void* dq, void* dk, void* dv, float* dW1,
                                float* dW3, float* dW2, void* workspace, size_t workspace_bytes, void* stream) {
  if (options == nullptr) return TTT_ERR_ARG;
  const int order = options->order;
  if ((options->loss != 0 && options->loss != 1) || (options->weight_norm != 0 && options->weight_norm != 1) ||
      (options->muon != 0 && options->muon != 1))
    return TTT_ERR_ARG;
  // the variants of the update itself have no backward here
  if (options->eta_tok != nullptr || options->loss != 0 || options->weight_norm != 0 || options->muon != 0)
    return TTT_ERR_UNSUPPORTED;
  int st = check_lact(shape, dtype);
  if (st != TTT_OK) return st;
  if (order != TTT_UPDATE_THEN_APPLY && order != TTT_APPLY_THEN_UPDATE) return TTT_ERR_ARG;
  if (!finite(eta)) return TTT_ERR_ARG;
  const int B = (int)shape->batch, H = (int)shape->heads, n = (int)shape->seq_len, dh = (int)shape->head_dim,
            m = (int)shape->hidden, C = (int)shape->chunk;
  if (H > 0 && (!ok_ptr(W1) || !ok_ptr(W3) || !ok_ptr(W2) || !ok_ptr(dW1) || !ok_ptr(dW3) || !ok_ptr(dW2)))
    return TTT_ERR_ARG;
  if ((int64_t)B * H * n > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(dO) || !ok_ptr(dq) ||
                                 !ok_ptr(dk) || !ok_ptr(dv)))
    return TTT_ERR_ARG;
  const bool saved = options->W_states != nullptr;
  if (saved && !aligned16(options->W_states)) return TTT_ERR_ARG;
  const size_t need = dtype == TTT_BF16 ? ttt::lact_bwd_workspace_bytes<bf16>(B, H, n, dh, m, C, saved)
                                        : ttt::lact_bwd_workspace_bytes<float>(B, H, n, dh, m, C, saved);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)) return TTT_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (H == 0) return TTT_OK;
  if (B == 0) {                    // no row: every weight gradient is zero
    const int64_t md = (int64_t)m * dh * H;
    int r = dev(ttt::launch_zero<float>(dW1, md, s));
    if (r == TTT_OK) r = dev(ttt::launch_zero<float>(dW3, md, s));
    if (r == TTT_OK) r = dev(ttt::launch_zero<float>(dW2, md, s));
    return r;
  }
  ttt::LactBwdArgs a{B, H, n, dh, m, C, order, eta, q, k, v, W1, W3, W2, dO, dq, dk, dv, dW1, dW3, dW2,
                     (char*)workspace, options->update_mask, options->W_states};
  return dev(dtype == TTT_BF16 ? ttt::launch_lact_backward<bf16>(a, s) : ttt::launch_lact_backward<float>(a, s));
}

int ttt_lact_swiglu_ex(const ttt_lact_shape* shape, int dtype, float eta, const void* q, const void* k, const void* v,
                       const void* W1, const void* W3, const void* W2, const ttt_lact_options* options, void* O,
                       float* W1_f, float* W3_f, float* W2_f, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (options == nullptr) return TTT_ERR_ARG;
  const int order = options->order;
  if ((options->loss != 0 && options->loss != 1) || (options->weight_norm != 0 && options->weight_norm != 1) ||
      (options->muon != 0 && options->muon != 1))
    return TTT_ERR_ARG;
  if (options->eta_tok != nullptr && !ok_ptr(options->eta_tok)) return TTT_ERR_ARG;
  if (options->side_stream != nullptr && (options->fork_event == nullptr || options->join_event == nullptr))
    return TTT_ERR_ARG;
  if (options->W_states != nullptr && !aligned16(options->W_states)) return TTT_ERR_ARG;
  int st = check_lact(shape, dtype);
  if (st != TTT_OK) return st;
  if (order != TTT_UPDATE_THEN_APPLY && order != TTT_APPLY_THEN_UPDATE) return TTT_ERR_ARG;
  if (!finite(eta)) return TTT_ERR_ARG;
  const int B = (int)shape->batch, H = (int)shape->heads, n = (int)shape->seq_len, dh = (int)shape->head_dim,
            m = (int)shape->hidden, C = (int)shape->chunk;
  if (B == 0) return TTT_OK;
  if (!ok_ptr(W1) || !ok_ptr(W3) || !ok_ptr(W2) || !ok_ptr(W1_f) || !ok_ptr(W3_f) || !ok_ptr(W2_f))
    return TTT_ERR_ARG;
  if (n > 0 && (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(O))) return TTT_ERR_ARG;
  const size_t need = dtype == TTT_BF16 ? ttt::lact_workspace_bytes<bf16>(B, H, n, dh, m, C)
                                        : ttt::lact_workspace_bytes<float>(B, H, n, dh, m, C);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)) return TTT_ERR_WORKSPACE;
  ttt::LactArgs a{B, H, n, dh, m, C, order, eta, q, k, v, W1, W3, W2, O, W1_f, W3_f, W2_f, (char*)workspace,
                  options->update_mask, options->eta_tok, options->loss, options->weight_norm, options->muon,
                  (hipStream_t)options->side_stream, (hipEvent_t)options->fork_event,
                  (hipEvent_t)options->join_event};
  a.keep = options->W_states;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == TTT_BF16 ? ttt::launch_lact<bf16>(a, s) : ttt::launch_lact<float>(a, s);
  if (e == hipErrorNotSupported) return TTT_ERR_UNSUPPORTED;
  return dev(e);
}

}  // extern "C"
