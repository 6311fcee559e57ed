// MFMA tile engine for gfx950 (CDNA4), shared by every contraction of the layer.
//
// A workgroup of 256 threads (4 waves of 64) owns a 256 x BQ tile (BQ = 256
// or 128) acc[p][q] = sum_k P[p][k] * Q[q][k] and walks K in steps of 128
// bytes (64 bf16 or 32 fp32).  Both operands are K-contiguous in global
// memory.  Each wave owns a 128 x BQ/2 quarter: 4 x NQB 32x32 MFMA accumulator
// blocks (NQB = BQ / 64), 64 NQB fp32 per lane, allocated to AGPRs.
//
// Global -> LDS: buffer_load_dwordx4 ... lds (LDS DMA).  One instruction moves
// 64 lanes x 16 B = 8 rows x 128 B of a tile with no VGPR staging.  Out-of-range
// rows and the K tail are read through a per-lane offset past the buffer
// resource's range, which the hardware returns as zero: no branches.
//
// LDS layout of a tile: 256 rows of 128 B; the 16-byte chunk c of row r sits
// in slot c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive rows hit
// 8 different bank groups.  The DMA reaches this layout by letting lane L of an
// instruction fetch chunk (L & 7) ^ (L >> 3) of its row.  Two stages of
// (256 + 256) x 128 B = 128 KB: step k+1 is in flight while step k is
// multiplied; one barrier per step (LDS: 2 x (256 + BQ) x 128 B).
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, or 4 x v_mfma_f32_32x32x2_f32 for
// fp32): P feeds the instruction's A slot, Q its B slot.  A lane therefore
// holds one q index and, per group of 4 registers, 4 consecutive p indices, so
// epilogues store 4 consecutive p values at once: whichever output dimension
// is contiguous in memory is mapped to P.
#pragma once
#include "common.hpp"

namespace ttt {

// GEMM kernels hold 256 accumulators per lane in AGPRs, which caps occupancy at
// one wave per SIMD anyway; saying so lets the scheduler spend registers on
// keeping LDS fragment reads ahead of the MFMAs instead of minimising them.
#define TTT_ONE_WAVE __attribute__((amdgpu_waves_per_eu(1, 1)))

constexpr int kThreads = 256;
constexpr int kTile = 256;                  // rows of the P tile
constexpr int kTileBytes = kTile * 128;     // bytes of one P tile stage
constexpr int kSmemBytes = 2 * (kTile + kTile) * 128;   // enough for either tile shape

// Stage layout for a 256 x BQ tile: P tile then Q tile.
template <int NQB> struct TileShape {
  static constexpr int BQ = 64 * NQB;
  static constexpr int kQBytes = BQ * 128;
  static constexpr int kStage = kTileBytes + kQBytes;
  static constexpr int kSmem = 2 * kStage;
};
constexpr unsigned kOOB = 0x80000000u;     // any offset >= this is outside every resource

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// ---------------------------------------------------------------- tile scheduling

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Renumber so
// that each XCD receives a contiguous range of logical tile ids: neighbouring
// tiles (which share operand rows) then share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int full = total & ~7;
  if (bid >= full) return bid;
  return (bid & 7) * (full >> 3) + (bid >> 3);
}

// Grouped raster over a TP x TQ grid: groups of G q-tiles, p fastest inside a
// group, so a run of consecutive ids covers a compact block of tiles.
__device__ __forceinline__ void grouped_tile(int id, int TP, int TQ, int G, int& tp, int& tq) {
  const int per_group = G * TP;
  const int g = id / per_group;
  const int r = id - g * per_group;
  const int rows = min(G, TQ - g * G);
  tq = g * G + r % rows;
  tp = r / rows;
}

// ---------------------------------------------------------------- LDS DMA operands

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const unsigned n = bytes >= (uint64_t)kOOB ? kOOB - 1u : (unsigned)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Byte offset, inside a 128-byte row, of the chunk this lane fetches.
__device__ __forceinline__ unsigned dma_chunk_bytes() {
  const unsigned L = threadIdx.x & 63u;
  return ((L & 7u) ^ (L >> 3)) << 4;
}

// K-contiguous operand moved by DMA into a ROWS-row tile.  Plain: instruction
// i of wave w fills tile rows (ROWS/4) w + 8 i + (0..7) from consecutive rows of
// one matrix.  DUAL (ROWS = 256): rows come in 32-row blocks alternating between
// two matrices (instructions 0..3 read the first, 4..7 the second), block pair
// w holding rows 32 w + (0..31) of both.
template <bool DUAL, int ROWS = 256>
struct DmaOp {
  static constexpr int NI = ROWS / 32;      // DMA instructions per wave
  static_assert(!DUAL || ROWS == 256, "dual operands fill 256-row tiles");
  __amdgpu_buffer_rsrc_t rs0, rs1;
  unsigned off[DUAL ? 4 : NI];
  unsigned kbytes;

  // rows_valid: rows of this tile inside the matrix; ld_bytes: row pitch.
  __device__ __forceinline__ void init(const void* base0, const void* base1, int rows_valid, uint64_t ld_bytes,
                                       unsigned kbytes_) {
    kbytes = kbytes_;
    const int w = threadIdx.x >> 6, L = threadIdx.x & 63;
    const uint64_t span = rows_valid > 0 ? (uint64_t)(rows_valid - 1) * ld_bytes + kbytes_ : 0;
    rs0 = make_rsrc(base0, span);
    rs1 = make_rsrc(DUAL ? base1 : base0, span);
#pragma unroll
    for (int i = 0; i < (DUAL ? 4 : NI); ++i) {
      const int r = DUAL ? w * 32 + i * 8 + (L >> 3) : w * (ROWS / 4) + i * 8 + (L >> 3);
      off[i] = r < rows_valid ? (unsigned)(r * ld_bytes) : kOOB;
    }
  }
  __device__ __forceinline__ void issue(int ks, char* tile) const {
    const unsigned kb = (unsigned)ks * 128u + dma_chunk_bytes();
    const bool kin = kb < kbytes;
    char* base = tile + (threadIdx.x >> 6) * NI * 1024;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const unsigned o = DUAL ? off[i & 3] : off[i];
      const unsigned voff = kin ? o + kb : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds((DUAL && i >= 4) ? rs1 : rs0, (lds_ptr_t)(base + i * 1024), 16, voff,
                                               0, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

template <int NQB>
__device__ __forceinline__ void load_frags(const char* tp, const char* tq, int g, u32x4 (&pf)[4], u32x4 (&qf)[NQB]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int prow = (w >> 1) * 128 + (lane & 31);
  const int qrow = (w & 1) * (32 * NQB) + (lane & 31);
  const int chunk = 2 * g + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) pf[i] = *reinterpret_cast<const u32x4*>(tp + lds_off(prow + 32 * i, chunk));
#pragma unroll
  for (int j = 0; j < NQB; ++j) qf[j] = *reinterpret_cast<const u32x4*>(tq + lds_off(qrow + 32 * j, chunk));
}

// One K step (four groups of 16 k for bf16 / 8 k for fp32).  Fragments are
// double-buffered in registers: the LDS reads of group g + 1 are issued before
// the MFMAs of group g, and scheduling fences keep the compiler from sinking
// them back next to their use.
template <typename T, int NQB>
__device__ __forceinline__ void compute_stage(const char* tp, const char* tq, f32x16 (&acc)[4][NQB]) {
  u32x4 pf[2][4], qf[2][NQB];
  load_frags<NQB>(tp, tq, 0, pf[0], qf[0]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int cur = g & 1;
    if (g < 3) load_frags<NQB>(tp, tq, g + 1, pf[cur ^ 1], qf[cur ^ 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NQB; ++j) mma(acc[i][j], pf[cur][i], qf[cur][j], (T*)nullptr);
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct NoHook {
  template <int NQB>
  __device__ __forceinline__ void operator()(int, f32x16 (&)[4][NQB]) const {}
};

template <int NQB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][NQB]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NQB; ++j) acc[i][j] = (f32x16){};
}

// nks steps over K.  hook(ks, acc) runs after step ks, past the barrier; it
// may read and write global memory but not LDS.
template <typename T, int NQB, class OP, class OQ, class Hook>
__device__ __forceinline__ void mainloop(const OP& op, const OQ& oq, int nks, f32x16 (&acc)[4][NQB], char* smem,
                                         const Hook& hook) {
  using S = TileShape<NQB>;
  if (nks <= 0) return;
  op.issue(0, smem);
  oq.issue(0, smem + kTileBytes);
  wait_dma();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    char* cur = smem + (ks & 1) * S::kStage;
    char* nxt = smem + ((ks & 1) ^ 1) * S::kStage;
    if (ks + 1 < nks) {
      op.issue(ks + 1, nxt);
      oq.issue(ks + 1, nxt + kTileBytes);
    }
    compute_stage<T, NQB>(cur, cur + kTileBytes, acc);
    wait_dma();
    __syncthreads();
    hook(ks, acc);
  }
}

// Coordinates of this lane's accumulator values inside the tile: block (i, j),
// register group g covers p = acc_p(i, g) + 0..3 at q = acc_q(j).
__device__ __forceinline__ int acc_p(int i, int g) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w >> 1) * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
}
template <int NQB = 4>
__device__ __forceinline__ int acc_q(int j) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return (w & 1) * (32 * NQB) + j * 32 + (lane & 31);
}

}  // namespace ttt
