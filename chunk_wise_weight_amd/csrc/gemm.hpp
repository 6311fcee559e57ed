// MFMA tile engine for gfx950 (CDNA4), shared by every contraction of the layer.
//
// A workgroup of 256 threads (4 waves of 64) owns a 256 x 256 output tile
// acc[p][q] = sum_k P[p][k] * Q[q][k] and walks K in steps of 128 bytes
// (64 bf16 or 32 fp32).  Each wave owns a 128 x 128 quarter held in 16
// 32x32 MFMA accumulator blocks (256 fp32 per lane, allocated to AGPRs).
//
// Both operands are staged in LDS in one layout: ROWS rows of 128 bytes, the
// 16-byte chunk c of row r stored at slot c ^ (r & 7), so that the 16-byte
// fragment reads of 8 consecutive rows hit 8 different bank groups.  Two
// stages of (256 + 256) x 128 B = 128 KB: global loads for step k+1 are in
// flight (in registers) while step k is multiplied, then written to the other
// stage; one barrier per step.
//
// Global operands come in two layouts, chosen per operand:
//   * K-contiguous  (element (row, k) at base[row * ld + k]) -- copied as is;
//   * MN-contiguous (element (row, k) at base[k * ld + row]) -- each thread
//     loads a V x V block (V = elements per 16 B) and transposes it in
//     registers before the LDS write, so the MFMA always reads K-packed rows.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, or 4 x v_mfma_f32_32x32x2_f32 for
// fp32): the P operand feeds the instruction's A slot, Q its B slot, so a lane
// ends up with one q index and, per group of 4 registers, 4 consecutive p
// indices.  Epilogues therefore write 4 consecutive p values per store: the
// output dimension that must be contiguous in memory is always mapped to P.
#pragma once
#include "common.hpp"

namespace ttt {

constexpr int kThreads = 256;
constexpr int kTile = 256;          // rows of P and of Q per workgroup
constexpr int kTileBytes = kTile * 128;
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kSmemBytes = 2 * kStageBytes;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// ---------------------------------------------------------------- tile scheduling

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Renumber so
// that each XCD receives a contiguous range of logical tile ids: neighbouring
// tiles (which share operand rows) then share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  int full = total & ~7;
  if (bid >= full) return bid;
  return (bid & 7) * (full >> 3) + (bid >> 3);
}

// Grouped raster over a TP x TQ grid: groups of G q-tiles, p fastest inside a
// group, so consecutive ids cover a compact G x (ids/G) block.
__device__ __forceinline__ void grouped_tile(int id, int TP, int TQ, int G, int& tp, int& tq) {
  int per_group = G * TP;
  int g = id / per_group;
  int r = id - g * per_group;
  int rows = min(G, TQ - g * G);
  tq = g * G + r % rows;
  tp = r / rows;
}

// ---------------------------------------------------------------- operand loaders

// K-contiguous operand.  Thread t copies chunk (t & 7) of rows (t >> 3) + 32 i.
template <typename T>
struct LoadKC {
  static constexpr int V = Vec<T>::V;
  static constexpr int BK = 8 * V;
  static constexpr int N = kTile * 8 / kThreads;   // 8 chunks per thread
  u32x4 r[N];
  const T* rowp[N];   // row start, or nullptr outside the matrix
  int kc, kmax;

  // row_ptr(i) must return the start of tile row i (or nullptr).
  template <class RowPtr>
  __device__ __forceinline__ void init(RowPtr row_ptr, int K) {
    kc = threadIdx.x & 7;
    kmax = K;
#pragma unroll
    for (int i = 0; i < N; ++i) rowp[i] = row_ptr(i * 32 + (threadIdx.x >> 3));
  }
  __device__ __forceinline__ void load(int ks) {
    int k = ks * BK + kc * V;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      u32x4 v = (u32x4){0u, 0u, 0u, 0u};
      if (rowp[i] != nullptr && k < kmax) v = *reinterpret_cast<const u32x4*>(rowp[i] + k);
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(char* tile) const {
#pragma unroll
    for (int i = 0; i < N; ++i)
      *reinterpret_cast<u32x4*>(tile + lds_off(i * 32 + (threadIdx.x >> 3), kc)) = r[i];
  }
};

// Transpose a V x V block held as V rows of 16 bytes.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8]) {
  // bf16: element c of row s is half (c & 1) of word c >> 1.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unsigned a = in[2 * j][c >> 1], b = in[2 * j + 1][c >> 1];
      out[c][j] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[c][j] = in[j][c];
}

// MN-contiguous operand: element (row, k) at base[k * ld + row], rows < rows_valid.
template <typename T>
struct LoadMC {
  static constexpr int V = Vec<T>::V;
  static constexpr int BK = 8 * V;
  static constexpr int RB = kTile / V;             // V-blocks along the rows
  static constexpr int NB = 8 * RB / kThreads;     // blocks per thread (1 bf16, 2 fp32)
  u32x4 r[NB][V];
  const T* base;
  int64_t ld;
  int rows_valid, kmax;

  __device__ __forceinline__ void init(const T* b, int64_t ld_, int rows, int K) {
    base = b;
    ld = ld_;
    rows_valid = rows;
    kmax = K;
  }
  __device__ __forceinline__ void load(int ks) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      int id = threadIdx.x + kThreads * b;
      int pb = id % RB, kb = id / RB;
      int col = pb * V;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        int k = ks * BK + kb * V + v;
        u32x4 x = (u32x4){0u, 0u, 0u, 0u};
        if (col < rows_valid && k < kmax) x = *reinterpret_cast<const u32x4*>(base + (int64_t)k * ld + col);
        r[b][v] = x;
      }
    }
  }
  __device__ __forceinline__ void store(char* tile) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      int id = threadIdx.x + kThreads * b;
      int pb = id % RB, kb = id / RB;
      u32x4 t[V];
      transpose_block(r[b], t);
#pragma unroll
      for (int c = 0; c < V; ++c) *reinterpret_cast<u32x4*>(tile + lds_off(pb * V + c, kb)) = t[c];
    }
  }
};

// ---------------------------------------------------------------- MFMA step

__device__ __forceinline__ void mma(f32x16& acc, u32x4 p, u32x4 q, bf16*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, p), __builtin_bit_cast(bf16x8, q),
                                                acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, u32x4 p, u32x4 q, float*) {
  // Lane-half h holds k = 4h + e of this 8-wide group in element e: four
  // 32x32x2 steps, step e contracting {e, 4 + e}, cover all eight.
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(p[e]), __uint_as_float(q[e]), acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void compute_stage(const char* tp, const char* tq, f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int prow = (w >> 1) * 128 + (lane & 31);
  const int qrow = (w & 1) * 128 + (lane & 31);
  const int half = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x4 pf[4], qf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = *reinterpret_cast<const u32x4*>(tp + lds_off(prow + 32 * i, 2 * g + half));
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[j] = *reinterpret_cast<const u32x4*>(tq + lds_off(qrow + 32 * j, 2 * g + half));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma(acc[i][j], pf[i], qf[j], (T*)nullptr);
  }
}

struct NoHook {
  __device__ __forceinline__ void operator()(int, f32x16 (&)[4][4]) const {}
};

// The main loop: nks steps of BK over K.  hook(ks, acc) runs after step ks
// (after the barrier; it may touch global memory but not LDS).
template <typename T, class LP, class LQ, class Hook>
__device__ __forceinline__ void mainloop(LP& lp, LQ& lq, int nks, f32x16 (&acc)[4][4], char* smem,
                                         const Hook& hook) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  if (nks <= 0) return;
  lp.load(0);
  lq.load(0);
  lp.store(smem);
  lq.store(smem + kTileBytes);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    char* cur = smem + (ks & 1) * kStageBytes;
    char* nxt = smem + ((ks & 1) ^ 1) * kStageBytes;
    const bool more = ks + 1 < nks;
    if (more) {
      lp.load(ks + 1);
      lq.load(ks + 1);
    }
    compute_stage<T>(cur, cur + kTileBytes, acc);
    if (more) {
      lp.store(nxt);
      lq.store(nxt + kTileBytes);
    }
    __syncthreads();
    hook(ks, acc);
  }
}

// Coordinates of this lane's accumulator values: block (i, j), register group
// g covers p = p0 + pofs(i, g) + 0..3 at q = q0 + qofs(j).
__device__ __forceinline__ int acc_p(int i, int g) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w >> 1) * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
}
__device__ __forceinline__ int acc_q(int j) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w & 1) * 128 + j * 32 + (lane & 31);
}

}  // namespace ttt
