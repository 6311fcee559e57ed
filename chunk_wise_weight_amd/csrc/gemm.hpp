// MFMA tile engine for gfx950 (CDNA4), shared by every contraction of the layer.
//
// A workgroup of NW = WP x WQ waves owns a BP x BQ tile acc[p][q] =
// sum_k P[p][k] * Q[q][k] and walks K in steps of 128 bytes (64 bf16 or 32
// fp32).  An operand is K-contiguous in global memory (DmaOp) or MN-major,
// one k index per row (DmaOpMN, transposed in LDS).  Wave (wp, wq) owns
// NPB x NQB 16x16 MFMA accumulator blocks (BP = 16 NPB WP, BQ = 16 NQB WQ).
// Every kernel uses one shape:
//   Wide = 8 waves, 2 x 4, 8 x 4 blocks: 256 x 256 tile, 128 accumulators per
//          lane, two waves per SIMD so that one wave's LDS and barrier waits
//          are covered by the other's MFMAs.
//
// Per 64-element K step the eight waves read 192 KB of fragments from LDS and
// the DMA writes 64 KB into it, about as many LDS cycles as the step's MFMAs
// take: LDS bandwidth and the MFMA pipe bound the loop together.
//
// Global -> LDS: buffer_load_dwordx4 ... lds (LDS DMA).  One instruction moves
// 64 lanes x 16 B = 8 rows x 128 B of a tile with no VGPR staging.  Out-of-range
// rows and the K tail are read through a per-lane offset past the buffer
// resource's range, which the hardware returns as zero: no branches.
//
// LDS layout of a tile: rows of 128 B; the 16-byte chunk c of row r sits in
// slot c ^ ((r >> 1) & 7).  The LDS serves a 16-byte read for 16 lanes at a
// time across 64 four-byte banks (256 B); an MFMA fragment read has those 16
// lanes on 16 consecutive rows at one chunk, and (r & 1, slot) then takes 16
// different values, one per 16-byte bank group.  The DMA reaches this layout
// by letting lane L of an instruction fetch chunk (L & 7) ^ swizzle(row) of
// its row.  Two stages of (BP + BQ) x 128 B: step k+1 is in flight while step
// k is multiplied; one barrier per step.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, or 4 x v_mfma_f32_16x16x4_f32 for
// fp32): P feeds the instruction's A slot, Q its B slot.  Operand lane l holds
// row l & 15 of its block and the 16 bytes of chunk 4 g + (l >> 4) of the K
// step (group g = 0, 1).  The 16x16 shape is preferred to 32x32x16: it moves a
// quarter of the accumulator per instruction and sustains a higher MFMA rate
// on random data.  Result lane l holds 4 consecutive p indices at one q index,
// so epilogues store 4 consecutive p values at once: whichever output
// dimension is contiguous in memory is mapped to P.
#pragma once
#include "common.hpp"

namespace ttt {

constexpr unsigned kOOB = 0x80000000u;     // any offset >= this is outside every resource

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ lds_swz(row)) << 4); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <int WP_, int WQ_, int NPB_, int NQB_>
struct TileCfg {
  static constexpr int WP = WP_, WQ = WQ_, NPB = NPB_, NQB = NQB_;
  static constexpr int BM = 16;                 // MFMA block edge
  static constexpr int GPB = 1;                 // groups of 4 accumulators per block and lane
  using Frag = f32x4;                           // one block's accumulators in one lane
  static constexpr int NW = WP * WQ, NT = 64 * NW;
  static constexpr int BP = BM * NPB * WP, BQ = BM * NQB * WQ;
  static constexpr int PBytes = BP * 128, QBytes = BQ * 128;
  static constexpr int Stage = PBytes + QBytes, Smem = 2 * Stage;
  // tile coordinates of this lane's accumulators: block (i, j), register
  // group g covers p = acc_p(i, g) + 0..3 at q = acc_q(j)
  __device__ static __forceinline__ int acc_p(int i, int g) {
    return (wave_id() / WQ) * (BM * NPB) + i * BM + g * 8 + (lane_id() >> 4) * 4;
  }
  __device__ static __forceinline__ int acc_q(int j) { return (wave_id() % WQ) * (BM * NQB) + j * BM + (lane_id() & 15); }
};
using Wide = TileCfg<2, 4, 8, 4>;
// 128 x 128 tiles of 4 waves and 64 KB of LDS, two workgroups per CU: for
// launches with too few 256 x 256 tiles to fill the GPU.
using Half = TileCfg<2, 2, 4, 4>;

// Kernel attributes: NT threads, and the number of waves per SIMD the register
// budget is planned for (the scheduler then spends registers on keeping LDS
// fragment reads ahead of the MFMAs).
#define TTT_GEMM_KERNEL(C) \
  __global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NW / 4, C::NW / 4)))

// ---------------------------------------------------------------- tile scheduling

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Renumber so
// that each XCD receives a contiguous range of logical tile ids: neighbouring
// tiles (which share operand rows) then share one L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int full = total & ~7;
  if (bid >= full) return bid;
  return (bid & 7) * (full >> 3) + (bid >> 3);
}

// Group-synchronous order, for grids made of consecutive groups of `per` tiles
// that share operands within a group (a chunk's applies, a batch row's):
// XCD x takes the x-th eighth of every group, group after group, so that all
// XCDs work on the same group at any time and its operands stay in the
// last-level cache, while each XCD's concurrent tiles are still neighbours in
// the group's own order.  Used when per % 8 == 0 and an XCD's share of a group
// is at least 16 tiles; smaller shares scatter an XCD's concurrent tiles over
// several groups and lose more L2 reuse than they gain (the plain XCD order,
// where each XCD sweeps its own range of groups, is then faster).
__device__ __forceinline__ int group_sync_tile(int bid, int total, int per) {
  if ((per & 7) != 0 || per < 128) return xcd_remap(bid, total);
  const int px = per >> 3, i = bid >> 3;
  return (i / px) * per + (bid & 7) * px + (i % px);
}

// Runs of R consecutive tiles dealt round-robin to the XCDs: XCD x takes runs
// x, x + 8, x + 16, ...  At any time the GPU works on about 8 consecutive runs
// (one round of tiles when R is the CUs of an XCD), and the R tiles an XCD
// runs together are one run, which a grouped raster makes a compact block of
// tiles sharing operand rows in that XCD's L2.  A tail of fewer than 8 R tiles
// keeps the dispatch order.
__device__ __forceinline__ int xcd_runs(int bid, int total, int R) {
  const int full = total / (8 * R) * (8 * R);
  if (bid >= full) return bid;
  const int L = bid >> 3;
  return ((L / R) * 8 + (bid & 7)) * R + L % R;
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

// Buffer resource over [base, base + bytes).  Every base and extent used here
// is the same for the whole workgroup; reading the words through
// readfirstlane tells the compiler so, which keeps the resource in scalar
// registers (a value it cannot prove uniform -- e.g. one computed by a
// vector-ALU integer division -- would otherwise be wrapped in a per-lane
// loop around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const unsigned n = bytes >= (uint64_t)kOOB ? kOOB - 1u : (unsigned)bytes;
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // readfirstlane works on int: each half goes back through unsigned before it
  // is widened, so that bit 31 of the low half is not sign-extended into the
  // high half.
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
  const uint64_t ub = ((uint64_t)hi << 32) | (uint64_t)lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ub), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)n), 0x00020000);
}

// K-contiguous operand moved by DMA into a ROWS-row tile by NW waves: DMA
// instruction i of wave w fills tile rows 8 (NI w + i) + (0..7), NI = ROWS /
// (8 NW).  Plain: tile row r is matrix row r.  DUAL: tile rows come in 32-row
// blocks alternating between two matrices (even blocks from the first, odd
// from the second), block 2m + s holding rows 32 m + (0..31) of matrix s.
template <int NW, int ROWS, bool DUAL = false>
struct DmaOp {
  static constexpr int NI = ROWS / (8 * NW);
  static_assert(NI >= 1 && NI * 8 * NW == ROWS, "tile rows must split evenly over the waves");
  // DUAL: each wave's 8 NI rows must lie in one 32-row block, so that the
  // wave reads one matrix and holds a single resource
  static_assert(!DUAL || 32 % (8 * NI) == 0, "dual: each wave reads rows of one 32-row block");
  __amdgpu_buffer_rsrc_t rs;
  unsigned off[NI];    // this lane's row offset, or kOOB for rows outside the matrix
  unsigned coff;       // byte offset of the chunk this lane fetches within the K step (even 8-row blocks)
  unsigned kbytes;

  // rows_valid: rows of each source matrix inside this tile; ld_bytes: row pitch.
  __device__ __forceinline__ void init(const void* base0, const void* base1, int rows_valid, uint64_t ld_bytes,
                                       unsigned kbytes_) {
    kbytes = kbytes_;
    const int w = wave_id(), L = lane_id();
    const uint64_t span = rows_valid > 0 ? (uint64_t)(rows_valid - 1) * ld_bytes + kbytes_ : 0;
    // block of this wave's first row: even blocks come from base0, odd from base1
    const bool second = DUAL && ((((w * NI) * 8) >> 5) & 1);
    rs = make_rsrc(second ? base1 : base0, span);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (w * NI + i) * 8 + (L >> 3);
      const int mr = DUAL ? ((r >> 6) << 5) + (r & 31) : r;
      off[i] = mr < rows_valid ? (unsigned)(mr * ld_bytes) : kOOB;
    }
    // Row r = 8 b + (L >> 3) of 8-row block b has swizzle (r >> 1) & 7 =
    // 4 (b & 1) + (L >> 4): one base offset, flipped by 64 B in odd blocks.
    coff = (unsigned)(((L & 7) ^ (L >> 4)) << 4);
  }
  __device__ __forceinline__ void issue(int ks, char* tile) const {
    const int w = wave_id();
    char* base = tile + w * NI * 1024;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const unsigned kb = (unsigned)ks * 128u + (coff ^ ((unsigned)((w * NI + i) & 1) << 6));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + i * 1024), 16,
                                               kb < kbytes ? off[i] + kb : kOOB, 0, 0, 0);
    }
  }
  // Fragment of the 16 tile rows m0 + (0..15) for k group g: one 16-byte read.
  static constexpr int kReads = 1;                // LDS read instructions per fragment
  __device__ static __forceinline__ u32x4 frag(const char* t, int m0, int g) {
    const int lane = lane_id();
    return *reinterpret_cast<const u32x4*>(t + lds_off(m0 + (lane & 15), 4 * g + (lane >> 4)));
  }
};

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  It is reached through a
// restrict-qualified pointer so that it carries alias-scope metadata: without
// any, the compiler's wait insertion takes it to alias every LDS-DMA write in
// flight and holds it until the next stage's prefetch has landed (the ordinary
// fragment reads carry type-based alias information and are not held back).
// The stage it reads was completed by the previous step's DMA wait and barrier.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr16(const char* __restrict__ p) {
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p));
}

// MN-major operand: the matrix holds one k index per row (pitch ld_bytes) with
// the tile's COLS m indices contiguous, e.g. a token-contiguous copy read by a
// contraction over the other dimension.  A K step of KR = 128 / sizeof(T) rows
// lands in LDS as KR rows of RB = COLS * sizeof(T) bytes (the same 128 B per m
// index as the K-major layout), chunk c of row r in slot c ^ swz(r).
//
// Fragments come back in the K-major operand's register layout (lane l: m =
// m0 + (l & 15), k = 8 (l >> 4) + (0..7) of group g for bf16, 4 (l >> 4) +
// (0..3) for fp32):
//  - bf16: ds_read_b64_tr_b16 transposes, within each 16-lane group, the 16 x 4
//    matrix of 16-bit values the group's lanes address (lane j's 8 bytes are
//    its row j) into lane j <- column j: output lane j, element e is element
//    j & 3 of input lane 4 e + (j >> 2).  Input lane j of group h therefore
//    addresses k row 8 h + (j >> 2) at m0 + 4 (j & 3); a second read 4 rows
//    further down gives elements 4..7.  The LDS serves 32 lanes (256 B) per
//    cycle: rows {0..3, 8..11} + 32 g (or + 4) at one 32-byte span, which
//    swz(r) = 2 (r & 3) + 8 ((r >> 3) & 1) places in 8 different 32-byte
//    bank groups.
//  - fp32: four 4-byte reads of rows 16 g + 4 (l >> 4) + e at column m0 +
//    (l & 15); swz(r) = 4 ((r >> 2) & 3) puts the four 16-lane groups (rows 4
//    apart) in different 64-byte bank quarters.
// The DMA reaches the layout by letting lane L fetch chunk slot(L) ^ swz(row).
// The resource is rebuilt for every K step at that step's first row, so the
// matrix may span more than the 2 GiB one resource covers.
template <typename T, int NW, int COLS>
struct DmaOpMN {
  static constexpr int KR = 128 / (int)sizeof(T);       // k rows per K step
  static constexpr int RB = COLS * (int)sizeof(T);      // LDS bytes per k row
  static constexpr int RPI = 1024 / RB;                 // k rows per DMA instruction
  static constexpr int NI = KR / (RPI * NW);            // DMA instructions per wave and step
  static_assert(RPI >= 1 && RPI * RB == 1024 && NI >= 1 && NI * RPI * NW == KR, "one step splits evenly");
  static constexpr int EPP = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  const char* base;
  uint64_t ld;
  int krows;                                            // k rows of the matrix (K extent)
  unsigned off[NI];                                     // offset of this lane's chunk in its row of the step, or kOOB
  int row[NI];                                          // k row within the step

  __device__ static __forceinline__ int swz(int r) {
    return sizeof(T) == 2 ? 2 * (r & 3) + 8 * ((r >> 3) & 1) : 4 * ((r >> 2) & 3);
  }
  // cols_valid (a multiple of EPP): m indices inside the matrix; krows_: K extent.
  __device__ __forceinline__ void init(const void* base_, int cols_valid, uint64_t ld_bytes, int krows_) {
    base = static_cast<const char*>(base_);
    ld = ld_bytes;
    krows = krows_;
    const int w = wave_id(), L = lane_id();
    constexpr int LPR = 64 / RPI;                       // lanes per k row of an instruction
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      row[i] = (w * NI + i) * RPI + L / LPR;
      const int c = (L % LPR) ^ swz(row[i]);
      off[i] = c * EPP < cols_valid ? (unsigned)(row[i] * ld_bytes) + (unsigned)(c * 16) : kOOB;
    }
  }
  __device__ __forceinline__ void issue(int ks, char* tile) const {
    const int w = wave_id();
    const int k0 = ks * KR;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (uint64_t)k0 * ld, (uint64_t)KR * ld);
    char* dst = tile + w * NI * 1024;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + i * 1024), 16,
                                               k0 + row[i] < krows ? off[i] : kOOB, 0, 0, 0);
  }
  static constexpr int kReads = sizeof(T) == 2 ? 2 : 4;
  __device__ static __forceinline__ u32x4 frag(const char* t, int m0, int g) {
    const int lane = lane_id(), h = lane >> 4, j = lane & 15;
    if constexpr (sizeof(T) == 2) {
      const int r = 32 * g + 8 * h + (j >> 2);
      const int byte = 2 * m0 + 8 * (j & 3);
      const char* p = t + r * RB + ((((byte >> 4) ^ swz(r))) << 4) + (byte & 15);
      const s16x4 a = lds_read_tr16(p);
      const s16x4 b = lds_read_tr16(p + 4 * RB);      // swz(r + 4) == swz(r)
      const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
      return u32x4{ua[0], ua[1], ub[0], ub[1]};
    } else {
      const int r = 16 * g + 4 * h;                        // rows r .. r + 3, all with swizzle 4 h
      const int byte = 4 * (m0 + j);
      const char* p = t + r * RB + ((((byte >> 4) ^ swz(r))) << 4) + (byte & 15);
      return u32x4{*reinterpret_cast<const unsigned*>(p), *reinterpret_cast<const unsigned*>(p + RB),
                   *reinterpret_cast<const unsigned*>(p + 2 * RB), *reinterpret_cast<const unsigned*>(p + 3 * RB)};
    }
  }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------- MFMA step

__device__ __forceinline__ void mma(f32x4& acc, u32x4 p, u32x4 q, bf16*) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, p), __builtin_bit_cast(bf16x8, q),
                                                acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, u32x4 p, u32x4 q, float*) {
  // Lane quarter h holds k = 4h + e of this 16-wide group in element e: four
  // 16x16x4 steps, step e contracting {e, 4 + e, 8 + e, 12 + e}, cover all 16.
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(p[e]), __uint_as_float(q[e]), acc, 0, 0, 0);
}

template <class C, class OP, class OQ, class PF, class QF>
__device__ __forceinline__ void load_frags(const char* tp, const char* tq, int g, PF& pf, QF& qf) {
  const int w = wave_id();
  const int pm = (w / C::WQ) * (C::BM * C::NPB), qm = (w % C::WQ) * (C::BM * C::NQB);
#pragma unroll
  for (int i = 0; i < C::NPB; ++i) pf[i] = OP::frag(tp, pm + C::BM * i, g);
#pragma unroll
  for (int j = 0; j < C::NQB; ++j) qf[j] = OQ::frag(tq, qm + C::BM * j, g);
}

// One K step (two groups of 32 k for bf16 / 16 k for fp32).  Only group 0's
// fragments are read before the first MFMA; group 1's LDS reads are spread
// over group 0's MFMAs (two MFMAs, then one read; one and one when both
// operands take several reads per fragment), so that the eight waves of a
// workgroup, which leave the step barrier together, do not all stall on one
// burst of LDS reads.  Scheduling fences keep the compiler to that order.
template <typename T, class C, class OP, class OQ, class Acc>
__device__ __forceinline__ void compute_stage(const char* tp, const char* tq, Acc& acc) {
  constexpr int NR = C::NPB * OP::kReads + C::NQB * OQ::kReads;   // LDS reads per group
  constexpr int NM = C::NPB * C::NQB;              // MFMAs per group (x4 for fp32)
  constexpr int MPM = sizeof(T) == 2 ? 1 : 4;      // MFMA instructions per block and group
  constexpr int MPR = 2 * NR <= NM * MPM ? 2 : 1;  // MFMAs issued per group-1 read
  static_assert(MPR * NR <= NM * MPM, "enough MFMAs to cover the next group's reads");
  u32x4 pf[2][C::NPB], qf[2][C::NQB];
  load_frags<C, OP, OQ>(tp, tq, 0, pf[0], qf[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<C, OP, OQ>(tp, tq, 1, pf[1], qf[1]);
#pragma unroll
  for (int i = 0; i < C::NPB; ++i)
#pragma unroll
    for (int j = 0; j < C::NQB; ++j) mma(acc[i][j], pf[0][i], qf[0][j], (T*)nullptr);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);   // MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // 1 LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM * MPM - MPR * NR, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < C::NPB; ++i)
#pragma unroll
    for (int j = 0; j < C::NQB; ++j) mma(acc[i][j], pf[1][i], qf[1][j], (T*)nullptr);
  __builtin_amdgcn_sched_barrier(0);
}

struct NoHook {
  template <class A>
  __device__ __forceinline__ void operator()(int, A&, char*) const {}
};

template <class C, class Acc>
__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < C::NPB; ++i)
#pragma unroll
    for (int j = 0; j < C::NQB; ++j) acc[i][j] = typename C::Frag{};
}

// nks steps over K.  hook(ks, acc, free_stage) runs after step ks, past the
// barrier, in every wave.  It may use the stage step ks was read from
// (C::Stage bytes at free_stage) -- the next write to it is the DMA issued at
// the start of step ks + 2 -- provided it ends with a barrier; other LDS is
// off limits.
template <typename T, class C, class OP, class OQ, class Hook, class Acc>
__device__ __forceinline__ void mainloop(const OP& op, const OQ& oq, int nks, Acc& acc, char* smem,
                                         const Hook& hook) {
  // The host compilation pass only needs the kernels' signatures; instantiating
  // this body there (target builtins, inline asm) trips template deduction.
#if defined(__HIP_DEVICE_COMPILE__)
  if (nks <= 0) return;
  op.issue(0, smem);
  oq.issue(0, smem + C::PBytes);
  wait_dma();
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    char* cur = smem + (ks & 1) * C::Stage;
    char* nxt = smem + ((ks & 1) ^ 1) * C::Stage;
    if (ks + 1 < nks) {
      op.issue(ks + 1, nxt);
      oq.issue(ks + 1, nxt + C::PBytes);
    }
    compute_stage<T, C, OP, OQ>(cur, cur + C::PBytes, acc);
    wait_dma();
    __syncthreads();
    hook(ks, acc, cur);
  }
#endif
}

// Steps k0 .. k1 - 1 only (the same loop, restarted at k0): a kernel may stop
// the K loop, work on the accumulators outside it, and continue.
template <typename T, class C, class OP, class OQ, class Hook, class Acc>
__device__ __forceinline__ void mainloop_range(const OP& op, const OQ& oq, int k0, int k1, Acc& acc, char* smem,
                                               const Hook& hook) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (k1 <= k0) return;
  op.issue(k0, smem);
  oq.issue(k0, smem + C::PBytes);
  wait_dma();
  __syncthreads();
  for (int ks = k0; ks < k1; ++ks) {
    const int i = ks - k0;
    char* cur = smem + (i & 1) * C::Stage;
    char* nxt = smem + ((i & 1) ^ 1) * C::Stage;
    if (ks + 1 < k1) {
      op.issue(ks + 1, nxt);
      oq.issue(ks + 1, nxt + C::PBytes);
    }
    compute_stage<T, C, OP, OQ>(cur, cur + C::PBytes, acc);
    wait_dma();
    __syncthreads();
    hook(ks, acc, cur);
  }
#endif
}

// ---------------------------------------------------------------- LDS-staged output

// After the K loop the operand stages are free.  An output tile is assembled
// there and copied out in whole 16-byte pieces along its rows, so that global
// stores cover full cache lines rather than the 32-byte runs one lane's
// accumulators map to.  Rows of COLS elements; piece c of row r sits at slot
// c ^ (r & 15), which spreads the column-wise puts of 16 consecutive rows
// over different banks.
template <typename TO, int COLS>
struct Staged {
  static constexpr int RB = COLS * (int)sizeof(TO);     // bytes per row
  static constexpr int PPR = RB / 16;                   // 16-byte pieces per row
  static constexpr int EPP = 16 / (int)sizeof(TO);      // elements per piece
  static_assert(PPR % 16 == 0, "rows of at least 16 pieces");
  char* base;

  __device__ __forceinline__ int off(int r, int col) const {
    const int byte = col * (int)sizeof(TO);
    return r * RB + ((((byte >> 4) ^ (r & 15))) << 4) + (byte & 15);
  }
  // elements col..col+3 of row r (col % 4 == 0: they share one piece)
  __device__ __forceinline__ void put4(int r, int col, float a, float b, float c, float d) const {
    store4(reinterpret_cast<TO*>(base + off(r, col)), a, b, c, d);
  }
  __device__ __forceinline__ void put1(int r, int col, float v) const {
    *reinterpret_cast<TO*>(base + off(r, col)) = from_f32<TO>(v);
  }
  // Rows [0, nrows) out to global memory, nrows <= MAXROWS (the rows the
  // staging area holds); dst(r, col) is the address of element col of row r
  // (col a multiple of EPP, 16-byte aligned) or nullptr to skip.  Thread x
  // copies piece x % PPR of rows x / PPR, x / PPR + NT / PPR, ...; it reads
  // BATCH of its pieces from LDS before storing any, so that one LDS wait
  // covers a batch (a loop of read, wait, store per piece leaves the wave
  // idle for the LDS latency at every piece).  A wave's stores cover whole
  // 128-byte lines.  STREAM: non-temporal stores, for data that is not read
  // again soon.  BATCH = 0: one piece at a time in a loop, for kernels that
  // keep their accumulators live across the copy-out and have no registers
  // to spare.
  template <int NT, int MAXROWS, bool STREAM = false, int BATCH = 8, class Dst>
  __device__ __forceinline__ void flush(int nrows, Dst&& dst) const {
    if constexpr (BATCH == 0) {
      for (int idx = threadIdx.x; idx < nrows * PPR; idx += NT) {
        const int r = idx / PPR, c = idx - r * PPR;
        TO* p = dst(r, c * EPP);
        if (p == nullptr) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + r * RB + ((c ^ (r & 15)) << 4));
        if constexpr (STREAM) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
        else *reinterpret_cast<u32x4*>(p) = v;
      }
    } else {
      static_assert(NT % PPR == 0, "a thread's pieces share one column slot");
      constexpr int RS = NT / PPR;                        // rows between a thread's pieces
      static_assert(MAXROWS % RS == 0, "whole rounds of pieces");
      constexpr int ITER = MAXROWS / RS;                  // pieces per thread
      constexpr int NB = BATCH < ITER ? BATCH : ITER;
      static_assert(ITER % NB == 0, "whole batches");
      const int c = (int)threadIdx.x % PPR, r0 = (int)threadIdx.x / PPR;
#pragma unroll
      for (int i0 = 0; i0 < ITER; i0 += NB) {
        u32x4 v[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int r = r0 + (i0 + u) * RS;
          v[u] = *reinterpret_cast<const u32x4*>(base + r * RB + ((c ^ (r & 15)) << 4));
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int r = r0 + (i0 + u) * RS;
          if (r >= nrows) continue;
          TO* p = dst(r, c * EPP);
          if (p == nullptr) continue;
          if constexpr (STREAM) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(p));
          else *reinterpret_cast<u32x4*>(p) = v[u];
        }
      }
    }
  }
  // Transposed copy-out: output row c (c < ncols) is column c of the staged
  // rows [0, nrows) (nrows a multiple of EPP); each 16-byte output piece
  // gathers EPP consecutive staged rows.  A wave covers 8 output rows x 8
  // pieces, so its stores form 128-byte runs.  dst(c, r) is the address of
  // output element r of row c, or nullptr to skip.
  template <int NT, class Dst>
  __device__ __forceinline__ void flush_t(int ncols, int nrows, Dst&& dst) const {
    const int ppc = nrows / EPP;                               // pieces per output row
    const int groups = (ncols + 7) / 8, chunks = (ppc + 7) / 8;
    for (int idx = threadIdx.x; idx < groups * chunks * 64; idx += NT) {
      const int lane = idx & 63, blk = idx >> 6;
      const int c = (blk / chunks) * 8 + (lane & 7), pc = (blk % chunks) * 8 + (lane >> 3);
      if (c >= ncols || pc >= ppc) continue;
      TO* p = dst(c, pc * EPP);
      if (p == nullptr) continue;
      TO v[EPP];
#pragma unroll
      for (int e = 0; e < EPP; ++e) v[e] = *reinterpret_cast<const TO*>(base + off(pc * EPP + e, c));
      *reinterpret_cast<u32x4*>(p) = *reinterpret_cast<const u32x4*>(v);
    }
  }
};

}  // namespace ttt
