// MFMA tile kernel for C <- alpha*A*B + beta*C, column-major, A and B not
// transposed, on gfx950 (CDNA4).  One template serves fp32 and fp64; the
// precision enters only through a trait that names the matrix instruction.
//
// Design (what the pages' techniques become on CDNA4):
//  * Shared-memory blocking of A and B ("optimizing-sgemm-on-nvidia-turing-
//    gpus", kernel 2 and the larger tiles of kernels 7-8; "HPC - Lecture 13",
//    section "Kernel 2: Shared Memory Optimization") becomes an LDS tile of
//    BM x BK of A and BK x BN of B per workgroup.
//  * 128-bit vector loads (the SGEMM study's float4 step; the "V3.
//    Vectorized and double buffer" page, measure (1)) become 16-byte global
//    loads (buffer loads with scalar descriptors and 32-bit lane offsets for
//    whole tiles) and 16-byte LDS reads and writes.
//  * Register micro-tiles and warp tiles (SGEMM study, kernels 5, 7 and 9)
//    become one wave-level tile of RB x CB matrix-core blocks whose
//    accumulators stay in registers for the whole K loop.
//  * Double buffering / prefetch (SGEMM study kernel 10; V3 page measure
//    (2)) becomes a ring of LDS stages: the next K tiles are fetched from HBM
//    into registers while the current one feeds the matrix cores, then
//    written to a free stage; one workgroup barrier per K tile.
//  * Bank-conflict fixes (V3 page, sections V3.1 and V3.2): column-major A
//    arrives m-contiguous and is stored as As[k][m] with no transpose, so its
//    16-byte writes and reads are contiguous per lane group; B arrives
//    k-contiguous and is stored as Bs[n][k] with an XOR swizzle of its 16-byte
//    chunks chosen so that the row-strided operand reads and the stores both
//    touch distinct banks.
//  * Edge tiles ("HPC - Lecture 13", kernel 2's note that a general version
//    must handle inactive threads): in the steady state, out-of-range rows
//    and columns are read from the tile's own first row or column (their
//    products only reach entries that are never stored); in the masked
//    loads, out-of-range rows, columns and K entries load as zero without
//    touching memory; stores are predicated.
//
// Operand permutations that let one 16-byte LDS read feed several MFMAs
// without changing the result:
//  * rows: within a super-block of W row blocks, MFMA row i of block b' is
//    tile row W*i + b', so lane l reads W consecutive rows of As at once;
//  * k: within a group of KG = KPER*V inner indices, the matrix instruction's
//    k slot g (lanes g*MB .. g*MB+MB-1) at step s takes inner index V*g + s,
//    so lane l reads V consecutive k of Bs at once.  A uses the same mapping,
//    so every product A(i,k)*B(k,j) is formed exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pgemm {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef double doublex2 __attribute__((ext_vector_type(2)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x2f32: 32x32 block, 2 inner indices per instruction.
struct TraitF32 {
  using T = float;
  using chunk_t = floatx4;           // one 16-byte chunk
  using acc_t = floatx16;            // accumulators of one block, per lane
  static constexpr int V = 4;        // elements per 16-byte chunk
  static constexpr int MB = 32;      // block edge
  static constexpr int KPER = 2;     // inner indices per instruction
  static constexpr int NACC = 16;    // accumulator elements per lane
  // Accumulator register r of lane l holds block row
  //   8*(r/4) + 4*(l/32) + r%4,  block column l%32
  // (measured on gfx950).  Registers come in runs of RUN_R consecutive rows;
  // run j of the lane with inner-index slot `kslot` starts at irow(j, kslot).
  static constexpr int RUN_R = 4;
  static __device__ __forceinline__ int irow(int run, int kslot) { return 8 * run + 4 * kslot; }
  static __device__ __forceinline__ acc_t mfma(T a, T b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f64_16x16x4f64: 16x16 block, 4 inner indices per instruction.
struct TraitF64 {
  using T = double;
  using chunk_t = doublex2;
  using acc_t = doublex4;
  static constexpr int V = 2;
  static constexpr int MB = 16;
  static constexpr int KPER = 4;
  static constexpr int NACC = 4;
  // Accumulator register r of lane l holds block row (l/16) + 4*r, block
  // column l%16 (measured on gfx950): runs of one row each.
  static constexpr int RUN_R = 1;
  static __device__ __forceinline__ int irow(int run, int kslot) { return kslot + 4 * run; }
  static __device__ __forceinline__ acc_t mfma(T a, T b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
};

template <typename T>
struct GemmArgs {
  int M, N, K;
  T alpha, beta;
  const T* A;
  const T* B;
  T* C;
  int lda, ldb, ldc;
  int tiles_m, tiles_n;
  int group_m;     // tile rows per raster group
  // Stream-K for the last, partly filled round of tiles (see sk_plan): the
  // first `full_tiles` tiles (in raster order) get one workgroup each; the
  // K tiles of the remaining ones are shared evenly by `sk_wgs` more
  // workgroups, which write raw partial sums to `ws` (full_tiles == all
  // tiles: no stream-K).
  int full_tiles;
  int sk_wgs;
  T* ws;
  // Nonzero when every offset of a whole-tile load from its tile's first
  // row/column fits a signed 32-bit byte count (see buffer_offsets_fit);
  // otherwise all tiles take the masked loads, with 64-bit addresses.
  int buf32;
  // Rows [M, M + strip_rows) of C below the tiles, computed by strip_wgs
  // more workgroups at the end of the grid (strip_rows_wg), in kernels
  // compiled with that role (STRIPF); 0 otherwise.
  int strip_rows;
  int strip_wgs;
  int strip_cgw;   // column groups per strip workgroup (strip_groups)
};

// Workgroup id -> linear tile id, for `count` workgroups.  The dispatcher
// hands consecutive workgroup ids to the 8 XCDs in turn, and each XCD has its
// own L2: give every XCD one contiguous range of tile ids.
__host__ __device__ inline int xcd_remap(int wg, int count) {
  const int xcd = wg & 7, local = wg >> 3;
  const int base = count >> 3, rem = count & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + local;
}

// Linear tile id -> (tile row, tile column), walking tiles in groups of
// `group_m` tile rows so that the workgroups resident on one XCD at the same
// time share A and B panels in its L2.
__host__ __device__ inline void raster(int t, int tiles_m, int tiles_n, int group_m, int& tm,
                                       int& tn) {
  const int per_group = group_m * tiles_n;
  const int group = t / per_group;
  const int first_m = group * group_m;
  const int gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int within = t - group * per_group;
  tm = first_m + within % gsize;
  tn = within / gsize;
}

// XOR swizzle of the 16-byte chunks of one Bs row (KC chunks per row), for
// matrix blocks of MB rows.  gfx950 serves a ds_read_b128 in four cycles of
// 16 lanes: 8-lane blocks b and b^3 (lanes 0-7 with 24-31, 8-15 with 16-23,
// 32-39 with 56-63, 40-47 with 48-55), and the 16 lanes of a cycle must fall
// in distinct 16-byte groups of a 256-byte bank line (measured with
// rocprofv3's SQ_LDS_BANK_CONFLICT).  An operand read has lane l on row
// (l % MB) at logical chunk c0 + l / MB; the swizzles below give every such
// cycle 16 distinct groups, and ds_write_b128 (8 lanes per cycle) fills
// whole rows, which is conflict-free for any XOR of the chunk index.
template <int KC, int MB>
__host__ __device__ inline int swz(int n) {
  if constexpr (KC == 4) {
    return (((n >> 1) ^ (n >> 3)) & 1) | (((n >> 2) & 1) << 1);
  } else if constexpr (KC == 8 && MB == 32) {
    return (n & 7) ^ ((n >> 3) & 1);
  } else if constexpr (KC == 16 && MB == 32) {
    // a row is a whole bank line: rows 0-7 with 24-31 and 8-15 with 16-23
    // (each read cycle's lanes) take 16 distinct chunk positions
    return n & 15;
  } else {
    static_assert(KC == 8 && MB == 16, "Bs rows of 4, 8 or 16 chunks; 16 x 16 or 32 x 32 blocks");
    return n & 7;
  }
}

template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS>
struct TileCfg {
  using T = typename TR::T;
  static constexpr int NT = WGM * WGN * 64 * KS;      // threads per workgroup
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int RB = WM / TR::MB, CB = WN / TR::MB;
  static constexpr int V = TR::V;
  static constexpr int W = RB < V ? RB : V;           // rows per lane per LDS read
  static constexpr int SB = RB / W;                   // row super-blocks
  static constexpr int KG = TR::KPER * V;             // inner indices per group
  static constexpr int KC = BK / V;                   // chunks per Bs row
  static constexpr int A_STAGE = BK * BM, B_STAGE = BN * BK;  // elements
  static constexpr int A_CHUNKS = A_STAGE / V, B_CHUNKS = B_STAGE / V;
  static constexpr int A_LOADS = A_CHUNKS / NT, B_LOADS = B_CHUNKS / NT;
  // Epilogue staging: one region of MB columns x WM rows per wave that
  // writes C (KS > 1: group 0 only); chunks XOR-swizzled within a column.
  static constexpr bool STAGED_EPI = sizeof(T) == 4;   // measured: fp64 gains nothing
  static constexpr int EPI_LDW = WM;
  static_assert(WM / V >= 8, "epilogue swizzle needs 8 chunks per column");
  static constexpr int EPI_ELEMS = STAGED_EPI ? WGM * WGN * TR::MB * EPI_LDW : 0;
  static constexpr int RING_ELEMS = STAGES * (A_STAGE + B_STAGE);
  static constexpr int LDS_ELEMS = RING_ELEMS > EPI_ELEMS ? RING_ELEMS : EPI_ELEMS;
  static constexpr int LDS_BYTES = LDS_ELEMS * (int)sizeof(T);
  // 32-bit registers per lane: accumulators, two operand sets, staging.
  static constexpr int ACC_REGS = RB * CB * TR::NACC * (int)sizeof(T) / 4;
  static constexpr int OPS_REGS = (CB * V + V * RB) * (int)sizeof(T) / 4;
  static constexpr int STAGE_REGS = (A_LOADS + B_LOADS) * 4;
  // Unroll the steady-state loop by the ring depth (compile-time stages, no
  // LDS address arithmetic) when that leaves room for the addresses it keeps
  // live; larger tiles would spill.
  static constexpr bool UNROLL = ACC_REGS + 2 * OPS_REGS + STAGE_REGS <= 192;
  // With beta != 0, the old C of a whole tile can be loaded into registers
  // during the last K tiles (one 16-byte chunk per lane and K tile, all but
  // the last) instead of in the epilogue, when that costs at most 32
  // registers: the staged
  // epilogue's chunks (MB columns x WM rows per column block, WM/V chunks
  // per column) of the CB column blocks, NPF_C chunks per lane.
  static constexpr int EPI_CPC = WM / V;
  static constexpr int EPI_NI = STAGED_EPI ? TR::MB * EPI_CPC / 64 : 1;
  static constexpr int NPF_C = CB * EPI_NI;
  static constexpr bool PF_C =
      STAGED_EPI && KS == 1 && UNROLL && STAGES > 2 && NPF_C * V * (int)sizeof(T) / 4 <= 32;
  // K tiles over which those loads are spread: whole trips of the unrolled
  // steady state
  static constexpr int PF_ITERS = (NPF_C + STAGES - 1) / STAGES * STAGES;
  // Direct-store epilogue with beta != 0: the tile's whole old C (one
  // element per accumulator, in the accumulators' layout) can be loaded into
  // registers once the K loop has issued its last global loads, when that
  // takes at most 64 registers.
  static constexpr bool PF_CT =
      !STAGED_EPI && KS == 1 && RB * CB * TR::NACC * (int)sizeof(T) / 4 <= 64;
  // The 64 x 64 classes (fp32 with one K group or two, fp64) store C
  // written through to memory (cache policy sc0 sc1) rather than leaving its
  // lines dirty in each XCD's L2.  Measured faster on the shapes they serve,
  // with beta = 0 and beta != 0: fp32 with one K group by up to 17 % at some
  // leading dimensions (see the staged epilogue), two K groups by up to
  // 0.6 %, fp64 by 1-2 % on single rounds.  Their stores address C from the
  // tile's first element with 32-bit byte offsets, so ldc is held to
  // WT_MAX_LDC (the host does not launch these classes beyond it).
  static constexpr bool WT_C = BM == 64 && BN == 64 && KS <= 2;
  static constexpr long long WT_MAX_LDC =
      WT_C ? (0x7fffffffLL / (long long)sizeof(T) - BM) / BN : 0;
  // When the grid also computes strip rows (one K group per strip
  // workgroup: its latency passes beside the tiles), the strip role's sums
  // per thread (at most STRIP_ACC elements, STRIP_SCMAX columns per wave)
  // must not take more registers than the tile role, or fewer tiles would
  // share a compute unit.
  // Waves per SIMD that the LDS allows (160 KiB per compute unit, NT/256
  // waves per SIMD per workgroup): the kernels with a strip role ask the
  // compiler to keep that occupancy (not their stream-K forms, whose own
  // piece loop already takes more registers than that occupancy leaves).
  static constexpr int LDS_OCC = (160 * 1024 / LDS_BYTES) * (NT / 256) > 8
                                     ? 8
                                     : (160 * 1024 / LDS_BYTES) * (NT / 256);
  static constexpr int STRIP_SCMAX = (sizeof(T) == 4 && BM >= 128) ? 8 : (sizeof(T) == 4 ? 4 : 2);
  static constexpr int STRIP_ACC = (sizeof(T) == 4 && BM >= 128) ? 16 : (sizeof(T) == 4 ? 8 : 4);
  static_assert(WM * WGM == BM && WN * WGN == BN, "waves tile the block");
  static_assert(RB * TR::MB == WM && CB * TR::MB == WN, "blocks tile the wave");
  static_assert(RB == 1 || RB == 2 || RB == 4 || RB == 8, "row blocks");
  static_assert(BK % KG == 0, "K tile is whole groups");
  static_assert(A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "even load split");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS per workgroup");
  static_assert(STAGES >= 2, "at least double buffering");
  static_assert(STAGES == 2 || (BK / KG / KS) % 2 == 0,
                "ring pipeline alternates two operand sets per wave's share of a tile");
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && STAGES > 2),
                "K split in two or four, ring pipeline only");
  // K split: groups 1 .. KS-1 pass their accumulators through LDS to group 0
  // at the end.
  static_assert(KS == 1 || (KS - 1) * (WGM * WGN) * RB * CB * TR::NACC * 64 <= LDS_ELEMS,
                "K-split hand-over fits in LDS");
};

// f(integral_constant<int, I>) for I = FIRST .. LAST-1, unrolled at compile
// time (so that an LDS stage index becomes an immediate offset).
template <int I, int LAST, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < LAST) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, LAST>(f);
  }
}

// Fused multiply-add in the element type: a*b + c rounded once to T.  (The
// generic __builtin_fma takes doubles: with float operands it would compute
// in double and round twice.)
__device__ __forceinline__ float fma_t(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_t(double a, double b, double c) { return __builtin_fma(a, b, c); }

// ---------------------------------------------------------------- loads
// 16 bytes at p.  VEC: p is 16-byte aligned.  Otherwise p is only element
// aligned; multi-dword global accesses on gfx950 need dword alignment only,
// so a byte copy of 16 bytes still becomes one global_load_dwordx4 (and one
// global_store_dwordx4 for stores).
template <class TR, bool VEC>
__device__ __forceinline__ typename TR::chunk_t load_chunk_full(const typename TR::T* p) {
  typename TR::chunk_t v;
  if constexpr (VEC) {
    v = *reinterpret_cast<const typename TR::chunk_t*>(p);
  } else {
    __builtin_memcpy(&v, p, sizeof(v));
  }
  return v;
}

template <class TR, bool VEC>
__device__ __forceinline__ void store_chunk(typename TR::T* p, typename TR::chunk_t v) {
  if constexpr (VEC) {
    *reinterpret_cast<typename TR::chunk_t*>(p) = v;
  } else {
    __builtin_memcpy(p, &v, sizeof(v));
  }
}

// One chunk of V consecutive elements starting at p; element e is in range
// when e < valid.  A whole chunk uses one 16-byte load; a partial chunk loads
// its in-range elements one by one; out-of-range elements are zero and are
// never read.
template <class TR, bool VEC>
__device__ __forceinline__ typename TR::chunk_t load_chunk(const typename TR::T* p, int valid) {
  using T = typename TR::T;
  typename TR::chunk_t v;
  if (valid >= TR::V) {
    v = load_chunk_full<TR, VEC>(p);
  } else {
#pragma unroll
    for (int e = 0; e < TR::V; ++e) v[e] = (e < valid) ? p[e] : T(0);
  }
  return v;
}

// Whole-tile loads go through a buffer resource (a scalar descriptor whose
// base is the tile's first element in the current K tile) with a 32-bit
// per-lane byte offset that stays the same for every K tile and a scalar
// offset per chunk.  The loop then spends no vector instructions on
// addresses and keeps no 64-bit pointers in registers.  Range checking is
// off (the record count is the maximum); every address is in bounds by
// construction.  The word-3 value selects 32-bit data for gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

template <class TR>
__device__ __forceinline__ typename TR::chunk_t load_chunk_buf(__amdgpu_buffer_rsrc_t r,
                                                               int voff, int soff) {
  return __builtin_bit_cast(typename TR::chunk_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// The same 16 bytes written straight to LDS: every lane of the wave writes
// at lds_wave (the same for all its lanes) + 16 * lane.
__device__ __forceinline__ void load_chunk_buf_lds(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                   void* lds_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_wave, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, kBufferWord3);
}

// 16 bytes stored at byte offset voff from the descriptor's base, written
// through to memory (cache policy sc0 sc1) instead of left dirty in L2.
template <class TR>
__device__ __forceinline__ void store_chunk_wt(__amdgpu_buffer_rsrc_t r, int voff,
                                               typename TR::chunk_t v) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, voff, 0, 17);
}

// Host check for GemmArgs::buf32: the largest byte offset of a whole-tile
// load from its descriptor base is below BK*lda + BM elements (A) and
// BN*ldb + BK elements (B).
template <typename T>
__host__ inline bool buffer_offsets_fit(int bm, int bn, int bk, long long lda, long long ldb) {
  const long long lim = 0x7fffffffLL / (long long)sizeof(T);
  return bk * lda + bm < lim && bn * ldb + bk < lim;
}

// Rows of C below the last whole tile row, when there are only a few of
// them: computing them as tiles would run a full tile's K loop for those
// rows.  Rows [i0, i0 + r) (r at most kStripRows) of a block of columns per
// workgroup of NT threads.  The NW waves form `cgw` groups of columns (each
// wave sums SCW columns) and NW/cgw groups along K; the launcher picks cgw
// so that there are at least as many workgroups as compute units, which
// spreads the strip's memory traffic evenly (beside tiles, a few heavy strip
// workgroups would slow the tiles they share a compute unit with).  With
// several column groups the strip of A passes through LDS in chunks of KC
// inner indices (staged once per workgroup, the r values of an inner index
// contiguous, and read by every column group); with one, each lane loads its
// own values of A directly.  A lane sums its inner indices in order, one fused
// multiply-add per step and the loads of U steps issued together; the lanes
// of a wave are then added by a butterfly of exchanges (which leaves the same
// total in every lane: each addition pairs the same two values on both
// lanes), and the K groups in order through LDS.  Deterministic.  The row
// count is a compile-time constant of the loop (one instance per r), so the
// sums take r x SCW registers.
constexpr int kStripRows = 8;

// Columns per wave for r rows: as many as keep the r x SCW sums within `acc`
// elements, at most sc_max.
__host__ __device__ constexpr int strip_cols(int r, int sc_max, int acc) {
  return acc / r < 1 ? 1 : (acc / r > sc_max ? sc_max : acc / r);
}

// Column groups per strip workgroup of nw waves, sc columns each, for n
// columns on `units` compute units: the most (a power of two dividing nw)
// that still leaves at least `units` workgroups, else 1.
__host__ __device__ inline int strip_groups(int n, int sc, int nw, int units) {
  int g = 1;
  while (g * 2 <= nw && nw % (g * 2) == 0 && (n + 2 * g * sc - 1) / (2 * g * sc) >= units) g *= 2;
  return g;
}

template <typename T, int NT, int SCW, int R, int LDSE>
__device__ __forceinline__ void strip_rows_r(const GemmArgs<T>& g, int i0, int wg, T* lds) {
  constexpr int NW = NT / 64;
  constexpr int PART = NW * R * SCW;             // K-group sums, after the chunk
  constexpr int KC = (LDSE - PART) / R / 64 * 64;
  static_assert(KC >= 64, "an A chunk covers a wave's lanes");
  constexpr int U = (R <= 2 && R * SCW * (int)sizeof(T) <= 32) ? 4 : 2;
  // wave-uniform (scalar) wave index and group counts, so that the column
  // addresses below stay in scalar registers and each load takes a 32-bit
  // lane offset
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int cgw = __builtin_amdgcn_readfirstlane(g.strip_cgw);
  const int cg = wave % cgw, kg = wave / cgw, kstep = 64 * (NW / cgw);
  const int j0 = (wg * cgw + cg) * SCW;          // this wave's first column
  const int nc = g.N - j0 < SCW ? g.N - j0 : SCW;  // its columns inside C (may be <= 0)
  T* const As = lds;                             // [KC][R]
  T* const part = lds + KC * R;                  // [NW][R][SCW]
  T acc[R][SCW];
#pragma unroll
  for (int q = 0; q < R; ++q)
#pragma unroll
    for (int c = 0; c < SCW; ++c) acc[q][c] = T(0);
  // Column c of this wave's B columns, clamped into C (N >= 1 here): every
  // load below is unconditional, so a step's loads issue together and one
  // wait covers them; the values of columns at or past N are then replaced
  // by zero (their sums are never stored).
  const T* bcol[SCW];
#pragma unroll
  for (int c = 0; c < SCW; ++c) {
    const int col = j0 + c < g.N ? j0 + c : g.N - 1;
    bcol[c] = g.B + (size_t)col * g.ldb;
  }
  if (cgw == 1) {
    // one column group: every inner index is used by one wave only, so each
    // lane loads its own values of A (the R rows of one inner index are
    // contiguous: one or two vector loads), with B's, U steps at a time
    const T* const arow = g.A + i0;
#pragma unroll U
    for (int k = kg * 64 + lane; k < g.K; k += kstep) {
      T b[SCW];
#pragma unroll
      for (int c = 0; c < SCW; ++c) {
        const T v = bcol[c][k];
        b[c] = c < nc ? v : T(0);
      }
      T a[R];
      __builtin_memcpy(a, arow + (size_t)k * g.lda, sizeof(a));
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int c = 0; c < SCW; ++c) acc[q][c] = fma_t(a[q], b[c], acc[q][c]);
    }
  } else {
  for (int k0 = 0; k0 < g.K; k0 += KC) {
    const int kc = g.K - k0 < KC ? g.K - k0 : KC;
    if (k0 > 0) __syncthreads();                 // every wave is done with the last chunk
    for (int e = t; e < kc * R; e += NT) {
      const int k = e / R, q = e - k * R;
      As[e] = g.A[(size_t)(k0 + k) * g.lda + i0 + q];
    }
    __syncthreads();
    if (nc > 0) {
#pragma unroll U
      for (int k = kg * 64 + lane; k < kc; k += kstep) {
        T b[SCW];
#pragma unroll
        for (int c = 0; c < SCW; ++c) {
          const T v = bcol[c][k0 + k];
          b[c] = c < nc ? v : T(0);
        }
        T a[R];
#pragma unroll
        for (int q = 0; q < R; ++q) a[q] = As[k * R + q];
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
          for (int c = 0; c < SCW; ++c) acc[q][c] = fma_t(a[q], b[c], acc[q][c]);
      }
    }
  }
  }
#pragma unroll
  for (int q = 0; q < R; ++q)
#pragma unroll
    for (int c = 0; c < SCW; ++c)
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[q][c] += __shfl_xor(acc[q][c], off, 64);
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int c = 0; c < SCW; ++c) part[(wave * R + q) * SCW + c] = acc[q][c];
  }
  __syncthreads();
  // thread (cg', q, c) adds the K groups' sums of its column in order
  const int kgw = NW / cgw;
  if (t < cgw * R * SCW) {
    const int g_ = t / (R * SCW), q = (t / SCW) % R, c = t % SCW;
    const int col = (wg * cgw + g_) * SCW + c;
    if (col < g.N) {
      T sum = part[(g_ * R + q) * SCW + c];
      for (int w = 1; w < kgw; ++w) sum += part[((w * cgw + g_) * R + q) * SCW + c];
      T* pc = g.C + (size_t)col * g.ldc + (i0 + q);
      T v = g.alpha * sum;
      if (g.beta != T(0)) v = fma_t(g.beta, *pc, v);
      *pc = v;
    }
  }
}

// The strip of r rows for workgroup `wg`, with LDSE elements of LDS at lds.
template <typename T, int NT, int SCMAX, int ACC, int LDSE>
__device__ __forceinline__ void strip_rows_wg(const GemmArgs<T>& g, int i0, int r, int wg,
                                              T* lds) {
  switch (r) {
#define PGEMM_STRIP_CASE(RR)                                                        \
  case RR:                                                                          \
    strip_rows_r<T, NT, strip_cols(RR, SCMAX, ACC), RR, LDSE>(g, i0, wg, lds);     \
    break;
    PGEMM_STRIP_CASE(1)
    PGEMM_STRIP_CASE(2)
    PGEMM_STRIP_CASE(3)
    PGEMM_STRIP_CASE(4)
    PGEMM_STRIP_CASE(5)
    PGEMM_STRIP_CASE(6)
    PGEMM_STRIP_CASE(7)
    default:
      strip_rows_r<T, NT, strip_cols(8, SCMAX, ACC), 8, LDSE>(g, i0, wg, lds);
      break;
#undef PGEMM_STRIP_CASE
  }
}

// ---------------------------------------------------------------- kernel
// SKP: the stream-K form (a workgroup may run two pieces, and pieces may go
// to the workspace); without it every workgroup is one whole tile into C.
// STRIPF: the last g.strip_wgs workgroups of the grid compute the rows below
// the tiles (strip_rows_wg) instead of a tile.  Being last, they are
// dispatched as the last round of tiles starts and run beside it on compute
// units whose LDS has room for a second workgroup, rather than after the
// whole grid as a kernel of their own would.
template <class TR, int BM, int BN, int BK, int WGM, int WGN, bool VEC, int STAGES, int KS,
          bool SKP, bool STRIPF = false>
__global__ void __launch_bounds__(WGM * WGN * 64 * KS) __attribute__((amdgpu_waves_per_eu(
    (STRIPF && !SKP) ? TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>::LDS_OCC : 1)))
gemm_tile_kernel(GemmArgs<typename TR::T> g) {
  using Cfg = TileCfg<TR, BM, BN, BK, WGM, WGN, VEC, STAGES, KS>;
  using T = typename TR::T;
  using chunk_t = typename TR::chunk_t;
  using acc_t = typename TR::acc_t;
  constexpr int V = TR::V, MB = TR::MB, NT = Cfg::NT;
  constexpr int RB = Cfg::RB, CB = Cfg::CB, W = Cfg::W, SB = Cfg::SB;
  constexpr int KG = Cfg::KG, KC = Cfg::KC;
  constexpr int A_LOADS = Cfg::A_LOADS, B_LOADS = Cfg::B_LOADS;

  // LDS: the A stages, then the B stages (so that, with a compile-time
  // stage, an access is one per-thread base plus an immediate offset).
  __shared__ __attribute__((aligned(16))) T lds[Cfg::LDS_ELEMS];

  if constexpr (STRIPF) {
    const int first = g.full_tiles + g.sk_wgs;
    if ((int)blockIdx.x >= first) {
      strip_rows_wg<T, NT, Cfg::STRIP_SCMAX, Cfg::STRIP_ACC, Cfg::LDS_ELEMS>(
          g, g.M, g.strip_rows, (int)blockIdx.x - first, lds);
      return;
    }
  }

  // Pieces of work of this workgroup: a tile, a range [kt_begin, kt_end) of
  // its K tiles and a destination (C, or a workspace slot for partial sums).
  // A workgroup of the full rounds has one piece: a whole tile into C.  The
  // stream-K workgroups (blockIdx >= full_tiles) share the K tiles of the
  // remaining tiles evenly: workgroup w takes iterations [w*I/P, (w+1)*I/P)
  // of the I = rest*nk iterations in (tile, K tile) order, which is the end
  // of one tile and the start of the next at most (P > rest, so a range is
  // shorter than a tile); piece j of workgroup w writes its raw partial sums
  // to workspace slot 2w + j.
  const int nk_all = (g.K + BK - 1) / BK;
  const bool sk_wg = SKP && (int)blockIdx.x >= g.full_tiles;
  const int w_sk = (int)blockIdx.x - g.full_tiles;
  long long sk_b0 = 0, sk_b1 = 0;
  int sk_r0 = 0, npieces = 1;
  if (sk_wg) {
    const long long rest = (long long)g.tiles_m * g.tiles_n - g.full_tiles;
    const long long iters = rest * nk_all;
    sk_b0 = (long long)w_sk * iters / g.sk_wgs;
    sk_b1 = (long long)(w_sk + 1) * iters / g.sk_wgs;
    sk_r0 = (int)(sk_b0 / nk_all);
    npieces = (sk_b1 > (long long)(sk_r0 + 1) * nk_all) ? 2 : 1;
  }
  auto tile_piece = [&](const int t_lin, const int kt_begin, const int kt_end,
                        const int slot) __attribute__((always_inline)) {
    int tm, tn;
    raster(t_lin, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // KS groups of WGM x WGN waves; every group covers the whole tile and takes
    // 1/KS of the inner-index groups of each K tile.
    const int kgrp = (KS == 1) ? 0 : wave / (WGM * WGN);
    const int wave_in = (KS == 1) ? wave : wave % (WGM * WGN);
    const int wrow = (wave_in % WGM) * Cfg::WM, wcol = (wave_in / WGM) * Cfg::WN;
    const int M = g.M, N = g.N, K = g.K;
    const int lda = g.lda, ldb = g.ldb;
    const bool full_mn = (m0 + BM <= M) && (n0 + BN <= N);

    // Per-thread load assignment.  Chunk q = tid + i*NT.
    //  A: column q / (BM/V), rows (q % (BM/V))*V .. +V-1 of the tile.
    //  B: column q / KC, inner indices (q % KC)*V .. +V-1 of the tile.
    chunk_t ra[A_LOADS], rb[B_LOADS];

    // Whole K tiles: unmasked buffer loads, no branches.  A thread's chunks
    // i = 0, 1, ... of a tile lie NT/(BM/V) columns of A apart, so A needs one
    // per-lane offset and a scalar step per chunk; each B chunk keeps its own
    // per-lane offset.  The descriptors move by whole K tiles (scalar work).
    // Tiles on the M or N edge take the same loads.  An A chunk whose rows
    // all lie at or beyond M, or a B column at or beyond N, only feeds entries
    // of C that are never stored, so it is read from the tile's first row /
    // column instead (in bounds; the values do not matter).  An A chunk that
    // straddles M (M not a multiple of V) is read whole: its elements past row
    // M-1 are the column's padding or, with a tight lda, the first V-2 rows of
    // the next column, and again only feed rows that are never stored.  Such
    // reads stay inside the (K-1)*lda + M elements of A when the column is not
    // the last one and lda >= V-1, so on the M edge the steady state stops
    // before the last column (k_whole) and the masked loads take the rest.
    static_assert(NT % (BM / V) == 0 && NT % KC == 0, "uniform steps between a thread's chunks");
    // Byte offsets from the tile's first row (A, in the tile's K tile) and
    // first column (B): A chunk i of tile kt is at a_off + i*a_step from
    // A + m0 + kt*BK*lda, B chunk i at b_off[i] from B + n0*ldb + kt*BK.
    // (Formed in 64 bits; they fit 32 when g.buf32 is set, and are unused
    // otherwise.)
    const int a_row = m0 + (tid % (BM / V)) * V;
    constexpr long long TS = sizeof(T);
    const int a_off =
        (int)(((long long)(tid / (BM / V)) * lda + (a_row < M ? a_row - m0 : 0)) * TS);
    constexpr int A_COLS = NT / (BM / V);   // columns of A between a thread's chunks
    const int a_step = (int)((long long)A_COLS * lda * TS);
    int b_off[B_LOADS];
  #pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int nn = tid / KC + i * (NT / KC);
      b_off[i] = (int)(((long long)(n0 + nn < N ? nn : 0) * ldb + (tid % KC) * V) * TS);
    }
    const T* const a_tile = g.A + m0;
    const T* const b_tile = g.B + (size_t)n0 * ldb;
    const bool straddle = (m0 + BM > M) && (M % V != 0);
    const bool edge_fast = !straddle || lda >= V - 1;
    const int k_whole = straddle ? (K - 1) / BK : K / BK;   // whole K tiles the loop may load
    auto gload_full = [&](int kt) {
      const __amdgpu_buffer_rsrc_t ar = tile_rsrc(a_tile + (size_t)kt * BK * (size_t)lda);
  #pragma unroll
      for (int i = 0; i < A_LOADS; ++i) ra[i] = load_chunk_buf<TR>(ar, a_off, i * a_step);
      const __amdgpu_buffer_rsrc_t br = tile_rsrc(b_tile + (size_t)kt * BK);
  #pragma unroll
      for (int i = 0; i < B_LOADS; ++i) rb[i] = load_chunk_buf<TR>(br, b_off[i], 0);
    };
    // Edge tiles and the K tail: out-of-range elements load as zero.
    auto gload_masked = [&](int kt) {
      const int k0 = kt * BK;
  #pragma unroll
      for (int i = 0; i < A_LOADS; ++i) {
        const int q = tid + i * NT;
        const int kk = q / (BM / V), mm = (q % (BM / V)) * V;
        const int k = k0 + kk, m = m0 + mm;
        const int valid = (k < K) ? min(M - m, V) : 0;
        if (valid > 0) ra[i] = load_chunk<TR, VEC>(g.A + (size_t)k * lda + m, valid);
        else ra[i] = chunk_t{};
      }
  #pragma unroll
      for (int i = 0; i < B_LOADS; ++i) {
        const int q = tid + i * NT;
        const int nn = q / KC, kk = (q % KC) * V;
        const int n = n0 + nn, k = k0 + kk;
        const int valid = (n < N) ? min(K - k, V) : 0;
        if (valid > 0) rb[i] = load_chunk<TR, VEC>(g.B + (size_t)n * ldb + k, valid);
        else rb[i] = chunk_t{};
      }
    };
    auto gload = [&](int kt) {
      if (g.buf32 && full_mn && (kt + 1) * BK <= K) gload_full(kt);
      else gload_masked(kt);
    };

    auto lstore = [&](int stage) {
      T* As = lds + stage * Cfg::A_STAGE;
      T* Bs = lds + STAGES * Cfg::A_STAGE + stage * Cfg::B_STAGE;
  #pragma unroll
      for (int i = 0; i < A_LOADS; ++i) {
        const int q = tid + i * NT;
        const int kk = q / (BM / V), mm = (q % (BM / V)) * V;
        *reinterpret_cast<chunk_t*>(As + kk * BM + mm) = ra[i];
      }
  #pragma unroll
      for (int i = 0; i < B_LOADS; ++i) {
        const int q = tid + i * NT;
        const int nn = q / KC, kc = q % KC;
        *reinterpret_cast<chunk_t*>(Bs + nn * BK + ((kc ^ swz<KC, TR::MB>(nn)) * V)) = rb[i];
      }
    };

    acc_t acc[RB][CB];
  #pragma unroll
    for (int b = 0; b < RB; ++b)
  #pragma unroll
      for (int c = 0; c < CB; ++c) acc[b][c] = acc_t{};

    // Lane roles in the matrix instruction.
    const int lrow = lane % MB;   // block row (A) / block column (B) of this lane
    const int kslot = lane / MB;  // which inner-index slot of the instruction

    // Old C of the tile, in the staged epilogue's layout: chunk q = c*NI + i
    // of this lane is rows rc*V .. rc*V+V-1 of column col of column block c
    // of the wave tile, with lane + 64*i = col*CPC + rc.  Loaded during the
    // last K tiles when beta != 0 and the whole tile lies inside C (pf_c),
    // one chunk per K tile, so that the reads of every tile's C spread over
    // the end of the K loop instead of all arriving in the epilogue at once.
    // The last chunk (three in the 128 x 128 kernel with strip workgroups,
    // which also holds the strip role's registers) waits for the epilogue:
    // fewer chunks held through the K loop keep the 128 x 128 kernels within
    // the 128 registers that leave room for a second workgroup per compute
    // unit.
    constexpr bool PF_C = Cfg::PF_C && !SKP;
    constexpr int NPF = PF_C ? Cfg::NPF_C : 1;
    constexpr int NPF_LATE = (STRIPF && BM >= 128 && NPF > 3) ? 3 : 1;
    chunk_t cpf[NPF];
    const bool pf_c = PF_C && slot < 0 && full_mn && g.beta != T(0);
    bool pf_done = false;
    // A lane's accumulator registers come in runs of RUN_R consecutive block
    // rows (see the trait).  Block b = sb*W + b' puts block row i at wave-tile
    // row sb*MB*W + W*i + b', so for fixed (c, sb, run) the lane owns RUN =
    // RUN_R*W consecutive rows of one column: element o of that run is
    // register run*RUN_R + o/W of block sb*W + o%W.
    constexpr int RUN = TR::RUN_R * W;
    constexpr int NRUN = TR::NACC / TR::RUN_R;
    // Direct-store epilogue: the old C of this lane's runs for group
    // gq = c*SB + sb, all of it loaded during the last K tiles (which read
    // only LDS) when beta != 0 and the whole tile lies inside C (ct_c).
    constexpr bool PF_CT = Cfg::PF_CT && !SKP;
    constexpr int NCT = PF_CT ? CB * SB : 1;
    T ct[NCT][NRUN][RUN];
    const bool ct_c = PF_CT && slot < 0 && full_mn && g.beta != T(0);
    bool ct_done = false;
    auto load_c_chunk = [&](const int q) __attribute__((always_inline)) {
      const int c = q / Cfg::EPI_NI, qq = lane + 64 * (q % Cfg::EPI_NI);
      const int col = qq / Cfg::EPI_CPC, rc = qq % Cfg::EPI_CPC;
      return load_chunk_full<TR, VEC>(g.C + (size_t)(n0 + wcol + c * MB + col) * g.ldc +
                                      (m0 + wrow + rc * V));
    };

    // Operands of one group of KG inner indices: CB chunks of B (V inner
    // indices each) and, for each of the V steps, the RB row values of A.
    struct GroupOps {
      chunk_t b[CB];
      T a[V][RB];
    };
    auto read_ops = [&](int stage, int kg, GroupOps& o) {
      const T* As = lds + stage * Cfg::A_STAGE;
      const T* Bs = lds + STAGES * Cfg::A_STAGE + stage * Cfg::B_STAGE;
  #pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int n = wcol + c * MB + lrow;
        const int kc = kg / V + kslot;
        o.b[c] = *reinterpret_cast<const chunk_t*>(Bs + n * BK + ((kc ^ swz<KC, TR::MB>(n)) * V));
      }
  #pragma unroll
      for (int s = 0; s < V; ++s) {
        const int k = kg + V * kslot + s;
  #pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const T* p = As + k * BM + wrow + sb * MB * W + W * lrow;
          if constexpr (W == 4) {
            floatx4 t = *reinterpret_cast<const floatx4*>(p);
  #pragma unroll
            for (int e = 0; e < 4; ++e) o.a[s][sb * W + e] = t[e];
          } else if constexpr (W == 2) {
            typedef T T2 __attribute__((ext_vector_type(2)));
            T2 t = *reinterpret_cast<const T2*>(p);
            o.a[s][sb * W + 0] = t[0];
            o.a[s][sb * W + 1] = t[1];
          } else {
            o.a[s][sb] = p[0];
          }
        }
      }
    };
    auto mma = [&](const GroupOps& o) {
  #pragma unroll
      for (int s = 0; s < V; ++s)
  #pragma unroll
        for (int b = 0; b < RB; ++b)
  #pragma unroll
          for (int c = 0; c < CB; ++c) acc[b][c] = TR::mfma(o.a[s][b], o.b[c][s], acc[b][c]);
    };

    constexpr int NG = BK / KG;      // inner-index groups per K tile
    constexpr int NGL = NG / KS;     // groups per K tile for one wave
    const int kg0 = kgrp * NGL * KG; // this wave's first inner index in a tile
    // This piece's K tiles: [kt_begin, kt_end) (all of them unless stream-K
    // workgroups share the tile).

    if constexpr (STAGES == 2) {
      // Two LDS stages.  Tile t+1 is fetched from HBM into registers while
      // tile t feeds the MFMAs, then written to the other stage; one barrier
      // per tile.  With one wave per SIMD (256 threads) the operands of group
      // g+1 are read into a second register set before the MFMAs of group g,
      // so LDS latency hides behind the same wave's matrix-core work; with more
      // waves per SIMD the other waves fill those gaps and one set is used.
      constexpr bool PIPE_OPS = NT <= 256;
      auto compute = [&](int stage) {
        if constexpr (PIPE_OPS) {
          GroupOps ops[2];
          read_ops(stage, 0, ops[0]);
  #pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            if (gi + 1 < NG) read_ops(stage, (gi + 1) * KG, ops[(gi + 1) & 1]);
            // keep the reads above the MFMAs (the scheduler would otherwise
            // sink each read next to its first use and wait for it there)
            __builtin_amdgcn_sched_barrier(0);
            mma(ops[gi & 1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
  #pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            GroupOps ops;
            read_ops(stage, gi * KG, ops);
            mma(ops);
          }
        }
      };
      gload(kt_begin);
      lstore(0);
      __syncthreads();
      for (int kt = kt_begin; kt < kt_end; ++kt) {
        const bool more = kt + 1 < kt_end;
        if (more) gload(kt + 1);
        compute((kt - kt_begin) & 1);
        if (more) lstore((kt + 1 - kt_begin) & 1);
        __syncthreads();
      }
    } else {
      // Ring of S = STAGES LDS stages, one barrier per tile.  At the top of
      // iteration kt the registers hold tile kt+S-1 (fetched one iteration
      // earlier, so HBM latency has a whole tile of MFMA work to hide behind);
      // they are written to stage (kt+S-1)%S, which last held tile kt-1 and was
      // released by the previous barrier, and tile kt+S is fetched.  The last
      // group of tile kt prefetches the operands of group 0 of tile kt+1, which
      // was written S-2 >= 1 barriers earlier, so the MFMAs of the next tile
      // start right after the barrier without waiting for LDS.
      constexpr int S = STAGES;
      constexpr int N_LD = A_LOADS + B_LOADS;                        // global loads
      // Tile kt's chunks straight from memory into LDS stage `stage` (buffer
      // loads to LDS: lane l of a wave writes 16 bytes at the wave's base +
      // 16*l, which is the stage layout of chunk q = tid + i*NT; for B the
      // lane loads the chunk that the swizzle puts at its place).  Whole K
      // tiles, with the redirected loads of gload_full on the M and N edges.
      auto dma_tile = [&](const int kt, const int stage) __attribute__((always_inline)) {
        const int wave_base = (tid & ~63) * V;   // elements
        T* As = lds + stage * Cfg::A_STAGE + wave_base;
        T* Bs = lds + STAGES * Cfg::A_STAGE + stage * Cfg::B_STAGE + wave_base;
        const __amdgpu_buffer_rsrc_t ar = tile_rsrc(a_tile + (size_t)kt * BK * (size_t)lda);
  #pragma unroll
        for (int i = 0; i < A_LOADS; ++i) load_chunk_buf_lds(ar, a_off, i * a_step, As + i * NT * V);
        const __amdgpu_buffer_rsrc_t br = tile_rsrc(b_tile + (size_t)kt * BK);
  #pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
          const int q = tid + i * NT, nn = q / KC;
          const int off = (int)(((long long)(n0 + nn < N ? nn : 0) * ldb +
                                 ((q % KC) ^ swz<KC, TR::MB>(nn)) * V) * TS);
          load_chunk_buf_lds(br, off, 0, Bs + i * NT * V);
        }
      };
      // The first S-1 tiles whole: all of them in flight at once with tile
      // S-1's register loads (one memory round trip before the first barrier
      // instead of one per stage).  Of the kernels with stream-K pieces only
      // the fp32 128 x 128 one: in the 64 x 64 ones it raises the registers
      // past their occupancy, and in fp64 it measured no gain.
      constexpr bool PRO_DMA = !SKP || (BM >= 128 && sizeof(T) == 4);
      if (PRO_DMA && g.buf32 && edge_fast && kt_begin + S - 1 <= min(kt_end, k_whole)) {
        for (int t = 0; t < S - 1; ++t) dma_tile(kt_begin + t, t);
        if (kt_begin + S - 1 < kt_end) gload(kt_begin + S - 1);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every stage has landed
        __syncthreads();
      } else {
        for (int t = 0; t < S - 1; ++t)
          if (kt_begin + t < kt_end) {
            gload(kt_begin + t);
            lstore(t);
          }
        if (kt_begin + S - 1 < kt_end) gload(kt_begin + S - 1);
        __syncthreads();
      }
      GroupOps ops[2];
      read_ops(0, kg0, ops[0]);
      // Drain those reads so that both edges into the loop header carry no
      // LDS operations in flight: otherwise the compiler's wait-count
      // insertion has to assume the prologue's reads are pending at every
      // iteration and makes the first MFMAs wait for the tile's LDS stores.
      // (s_waitcnt lgkmcnt(0); the vector-memory and export counts at their
      // no-wait maxima.)
      __builtin_amdgcn_s_waitcnt(0xC07F);
      // Instruction counts of one iteration, for the interleave below.
      constexpr int N_RD = CB + V * SB;                              // ds_read per group
      constexpr int N_WR = A_LOADS + B_LOADS;                        // ds_write
      constexpr int MPG = V * RB * CB;                                // MFMAs per group
      constexpr bool INTERLEAVE = NGL >= 2 && MPG >= N_WR + N_LD;
      // A group too short for both (BK 32 on 32 x 32 wave tiles): the stores
      // between group 0's MFMAs, the global loads between group 1's.
      constexpr bool SPLIT = !INTERLEAVE && NGL >= 2 && MPG >= N_WR && MPG >= N_LD;
      // Operand reads too, one between MFMAs, when a group has room for them.
      // After each barrier every wave starts the same group at once; reads
      // issued as a block then queue behind the other waves' reads, and both
      // waves of a SIMD stall with the matrix core idle.
      constexpr bool READS_SPREAD = MPG >= N_RD;
      constexpr bool RIL = INTERLEAVE && MPG >= N_RD + N_WR + N_LD;
      // Schedule: the operand reads of the next group one per MFMA, then the
      // rest of the group's MFMAs (groups without stores or loads).
      auto spread_reads = [&]() {
        if constexpr (READS_SPREAD) {
  #pragma unroll
          for (int i = 0; i < N_RD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, MPG - N_RD, 0);
        }
      };
      int st = 0;                       // stage of tile kt
      int kt = kt_begin;
      // Steady state, while tile kt+S exists and is whole (edge tiles too,
      // with the redirected loads above): one branch-free block per
      // iteration.  With in-order issue, the next group's operand reads, the
      // tile's LDS stores and its global loads are spread evenly between
      // group 0's MFMAs (each executes while an MFMA occupies the matrix
      // core) instead of running as a block while the matrix core idles.
      const int kt_fast_end = ((INTERLEAVE || SPLIT) && edge_fast && g.buf32)
                                  ? max(kt_begin, min(kt_end, k_whole) - S)
                                  : kt_begin;
      // The steady state is unrolled by S, so that every stage index is a
      // compile-time constant and each LDS access is a per-thread base plus an
      // immediate offset (no address arithmetic per iteration).
      // qc: the chunk of old C this iteration loads (-1: none).
      auto fast_iteration = [&](const int st, const int kt, auto qc) __attribute__((always_inline)) {
        constexpr int QC = decltype(qc)::value;
        const int st_next = (st + 1 == S) ? 0 : st + 1;
        const int st_store = (st == 0) ? S - 1 : st - 1;   // (kt + S - 1) % S
        read_ops(st, kg0 + KG, ops[1]);
        if constexpr (!RIL) __builtin_amdgcn_sched_barrier(0);
        lstore(st_store);
        if constexpr (!SPLIT) {
          gload_full(kt + S);
          // after the tile's own loads, so that waiting for those (in issue
          // order) never waits for this one
          if constexpr (QC >= 0) cpf[QC] = load_c_chunk(QC);
        }
        mma(ops[0]);
        if constexpr (SPLIT) {
          constexpr int SP = MPG / N_WR;
  #pragma unroll
          for (int i = 0; i < N_WR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
          }
          __builtin_amdgcn_sched_group_barrier(0x008, MPG - SP * N_WR, 0);
        }
        if constexpr (INTERLEAVE) {
          // spread evenly: SP MFMAs before each read, store and load
          constexpr int N_LDI = N_LD + ((QC >= 0 && MPG >= N_WR + N_LD + 1) ? 1 : 0);
          constexpr int NM = (RIL ? N_RD : 0) + N_WR + N_LDI;
          constexpr int SP = MPG / NM;
          if constexpr (RIL) {
  #pragma unroll
            for (int i = 0; i < N_RD; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            }
          }
  #pragma unroll
          for (int i = 0; i < N_WR; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
          }
  #pragma unroll
          for (int i = 0; i < N_LDI; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, MPG - SP * NM, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int gi = 1; gi < NGL; ++gi) {
          // the next tile (kt+1 < kt_fast_end + S <= kt_end) always exists here
          if (gi + 1 < NGL) read_ops(st, kg0 + (gi + 1) * KG, ops[(gi + 1) & 1]);
          else read_ops(st_next, kg0, ops[(gi + 1) & 1]);
          if (SPLIT && gi == 1) {
            __builtin_amdgcn_sched_barrier(0);
            gload_full(kt + S);
            if constexpr (QC >= 0) cpf[QC] = load_c_chunk(QC);
            mma(ops[gi & 1]);
            constexpr int N_LDI = N_LD + ((QC >= 0 && MPG >= N_LD + 1) ? 1 : 0);
            constexpr int SP = MPG / N_LDI;
  #pragma unroll
            for (int i = 0; i < N_LDI; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MPG - SP * N_LDI, 0);
          } else {
            if constexpr (!READS_SPREAD) __builtin_amdgcn_sched_barrier(0);
            mma(ops[gi & 1]);
            spread_reads();
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
      };
      // Old C for the direct-store epilogue (ct_c), issued by the second of
      // the last S tiles (in the drain below or the loop after it): the first
      // one's LDS stores have consumed every A and B load by then, so no wait
      // for those can also wait for these, and the remaining tiles (LDS reads
      // and MFMAs only, thousands of cycles each) hide their latency.
      auto load_ct = [&]() __attribute__((always_inline)) {
        if constexpr (PF_CT) {
          if (ct_c) {
            static_for<0, NCT>([&](auto gq_c) {
              constexpr int gq = decltype(gq_c)::value;
              constexpr int c = gq / SB, sb = gq % SB;
              const T* pcol = g.C + (size_t)(n0 + wcol + c * MB + lrow) * g.ldc;
              const int row0 = m0 + wrow + sb * MB * W;
  #pragma unroll
              for (int run = 0; run < NRUN; ++run) {
                const T* pc = pcol + row0 + W * TR::irow(run, kslot);
                if constexpr (RUN % V == 0) {
  #pragma unroll
                  for (int h = 0; h < RUN / V; ++h) {
                    chunk_t v = load_chunk_full<TR, VEC>(pc + h * V);
  #pragma unroll
                    for (int e = 0; e < V; ++e) ct[gq][run][h * V + e] = v[e];
                  }
                } else {
  #pragma unroll
                  for (int o = 0; o < RUN; ++o) ct[gq][run][o] = pc[o];
                }
              }
            });
            ct_done = true;
          }
        }
      };
      // The last S tiles when they are whole and the steady state ends at
      // stage 0 (K a multiple of S*BK on the fast path): the same iteration
      // without global loads, the first storing the last tile fetched, and
      // with compile-time stages like the steady state's (the general loop
      // below computes LDS addresses and branches at run time, ~15 % slower
      // per tile).
      auto drain_iteration = [&](auto st_c) __attribute__((always_inline)) {
        constexpr int st = decltype(st_c)::value;
        constexpr bool first = st == 0, last = st == S - 1;
        // the last tile's prefetch re-reads its own stage (in bounds, unused)
        constexpr int st_next = last ? st : st + 1;
        if constexpr (st == 1) load_ct();
        read_ops(st, kg0 + KG, ops[1]);
        if constexpr (!RIL) __builtin_amdgcn_sched_barrier(0);
        if constexpr (first) lstore(S - 1);
        mma(ops[0]);
        constexpr int N_WRD = first ? N_WR : 0;
        constexpr int NM = (RIL ? N_RD : 0) + N_WRD;
        if constexpr ((INTERLEAVE || SPLIT) && NM > 0) {
          constexpr int SP = MPG / NM;
          if constexpr (RIL) {
  #pragma unroll
            for (int i = 0; i < N_RD; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            }
          }
  #pragma unroll
          for (int i = 0; i < N_WRD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, SP, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
          }
          __builtin_amdgcn_sched_group_barrier(0x008, MPG - SP * NM, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int gi = 1; gi < NGL; ++gi) {
          if (gi + 1 < NGL) read_ops(st, kg0 + (gi + 1) * KG, ops[(gi + 1) & 1]);
          else read_ops(st_next, kg0, ops[(gi + 1) & 1]);
          if constexpr (!READS_SPREAD) __builtin_amdgcn_sched_barrier(0);
          mma(ops[gi & 1]);
          spread_reads();
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
      };
      using NoC = std::integral_constant<int, -1>;
      // st == 0 here (kt == kt_begin), and after every S iterations
      if constexpr (Cfg::UNROLL) {
        // With pf_c, the last PF_ITERS whole trips before kt_fast_end (or
        // later) load the old C, one chunk per iteration.
        constexpr int PI = Cfg::PF_ITERS;
        const bool pf_loop = pf_c && kt_fast_end - kt_begin >= PI;
        const int kt_main_end =
            pf_loop ? kt_begin + (kt_fast_end - kt_begin - PI) / S * S : kt_fast_end;
        for (; kt + S <= kt_main_end; kt += S)
          static_for<0, S>([&](auto st_c) {
            fast_iteration(decltype(st_c)::value, kt + decltype(st_c)::value, NoC{});
          });
        if constexpr (PF_C) {
          if (pf_loop) {
            static_for<0, PI / S>([&](auto trip) {
              static_for<0, S>([&](auto st_c) {
                constexpr int q = decltype(trip)::value * S + decltype(st_c)::value;
                fast_iteration(decltype(st_c)::value, kt + decltype(st_c)::value,
                               std::integral_constant<int, (q < NPF - NPF_LATE ? q : -1)>{});
              });
              kt += S;
            });
            pf_done = true;
          }
        }
      }
      for (; kt < kt_fast_end; ++kt) {
        fast_iteration(st, kt, NoC{});
        st = (st + 1 == S) ? 0 : st + 1;
      }
      if constexpr (Cfg::UNROLL) {
        if (st == 0 && kt == kt_fast_end && kt + S == kt_end && kt > kt_begin) {
          static_for<0, S>([&](auto st_c) { drain_iteration(st_c); });
          kt = kt_end;
        }
      }
      // Remaining iterations (edge tiles, the K tail, the last S tiles).
      for (; kt < kt_end; ++kt) {
        if constexpr (PF_CT) {
          if (kt == kt_end - S + 1) load_ct();
        }
        const int st_next = (st + 1 == S) ? 0 : st + 1;
        const int st_store = (st == 0) ? S - 1 : st - 1;   // (kt + S - 1) % S
        // At the last tile the prefetch re-reads this tile's own stage (in
        // bounds, unused): a branch here would make the compiler wait for the
        // prefetch before the current group's MFMAs.
        const int st_pf = (kt + 1 < kt_end) ? st_next : st;
        if (kt + S - 1 < kt_end) lstore(st_store);
        if (kt + S < kt_end) gload(kt + S);
  #pragma unroll
        for (int gi = 0; gi < NGL; ++gi) {
          if (gi + 1 < NGL) read_ops(st, kg0 + (gi + 1) * KG, ops[(gi + 1) & 1]);
          else read_ops(st_pf, kg0, ops[(gi + 1) & 1]);
          if constexpr (!READS_SPREAD) __builtin_amdgcn_sched_barrier(0);
          mma(ops[gi & 1]);
          spread_reads();
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        st = st_next;
      }
    }

    // K groups with one column block per wave: every wave stages its partial
    // sums in an LDS region of its own (group g, wave w), in the staged
    // epilogue's layout, and then every thread takes its share of the tile's
    // 16-byte chunks, adds the groups' values in group order (the same sums
    // as a hand-over to group 0) and stores them: no serial hand-over, and no
    // staging by group 0 alone while the other groups wait.
    constexpr bool PAR_EPI = KS > 1 && CB == 1 && Cfg::STAGED_EPI;
    if constexpr (PAR_EPI) {
      constexpr int NW = WGM * WGN;                // waves per group
      constexpr int LDW = Cfg::EPI_LDW;            // staging column stride (elements)
      constexpr int CPC = Cfg::WM / V;             // chunks per wave-tile column
      constexpr int WCH = MB * CPC;                // chunks per wave tile
      constexpr int PER = NW * WCH / NT;           // chunks per thread
      constexpr int RUN_E = TR::RUN_R * W, NRUN_E = TR::NACC / TR::RUN_R;
      static_assert(PER >= 1 && NW * WCH == PER * NT, "whole chunks per thread");
      static_assert(KS * NW * MB * LDW <= Cfg::LDS_ELEMS, "a staging region per wave");
      // Destination: C, or for a stream-K piece its raw partial sums (alpha
      // = 1, beta = 0, all BM x BN elements, column-major with ld = BM) in
      // workspace slot `slot`.
      const bool to_ws = slot >= 0;
      T* const cbase = to_ws ? g.ws + (size_t)slot * (BM * BN) : g.C;
      const int ldc = to_ws ? BM : g.ldc;
      const int m_end = to_ws ? BM : M, n_end = to_ws ? BN : N;
      const int r0 = to_ws ? 0 : m0, c0 = to_ws ? 0 : n0;
      const T alpha = to_ws ? T(1) : g.alpha, beta = to_ws ? T(0) : g.beta;
      const bool read_c = beta != T(0);
      // this thread's chunks: wave tile w, column col, rows rc*V .. rc*V+V-1
      int gcol[PER], grow[PER], loff[PER];
      chunk_t cold[PER];
  #pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int q = tid + i * NT;
        const int w = q / WCH, qq = q % WCH;
        const int col = qq / CPC, rc = qq % CPC;
        gcol[i] = c0 + (w / WGM) * Cfg::WN + col;
        grow[i] = r0 + (w % WGM) * Cfg::WM + rc * V;
        loff[i] = w * (MB * LDW) + col * LDW + (rc ^ (col & 7)) * V;
        cold[i] = chunk_t{};
        if (read_c && full_mn)
          cold[i] = load_chunk_full<TR, VEC>(cbase + (size_t)gcol[i] * ldc + grow[i]);
      }
      __syncthreads();                       // every wave is done with the ring
      T* const stg = lds + (kgrp * NW + wave_in) * (MB * LDW);
  #pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
  #pragma unroll
        for (int run = 0; run < NRUN_E; ++run) {
          T* const pcol = stg + lrow * LDW;
          const int ch0 = (sb * MB * W + W * TR::irow(run, kslot)) / V;
  #pragma unroll
          for (int h = 0; h < RUN_E / V; ++h) {
            chunk_t v;
  #pragma unroll
            for (int e = 0; e < V; ++e) {
              const int o = h * V + e;
              v[e] = acc[sb * W + o % W][0][run * TR::RUN_R + o / W];
            }
            *reinterpret_cast<chunk_t*>(pcol + ((ch0 + h) ^ (lrow & 7)) * V) = v;
          }
        }
      }
      __syncthreads();
  #pragma unroll
      for (int i = 0; i < PER; ++i) {
        chunk_t v = *reinterpret_cast<const chunk_t*>(lds + loff[i]);
  #pragma unroll
        for (int j = 1; j < KS; ++j) {
          const chunk_t p = *reinterpret_cast<const chunk_t*>(lds + j * (NW * MB * LDW) + loff[i]);
  #pragma unroll
          for (int e = 0; e < V; ++e) v[e] += p[e];
        }
        if (gcol[i] >= n_end) continue;
        T* const pc = cbase + (size_t)gcol[i] * ldc + grow[i];
        if (grow[i] + V <= m_end) {
          chunk_t out;
          if (read_c) {
            if (!full_mn) cold[i] = load_chunk_full<TR, VEC>(pc);
  #pragma unroll
            for (int e = 0; e < V; ++e) out[e] = fma_t(beta, cold[i][e], alpha * v[e]);
          } else {
  #pragma unroll
            for (int e = 0; e < V; ++e) out[e] = alpha * v[e];
          }
          if constexpr (Cfg::WT_C)
            store_chunk_wt<TR>(tile_rsrc(cbase + (size_t)c0 * ldc + r0),
                               ((gcol[i] - c0) * ldc + (grow[i] - r0)) * (int)sizeof(T), out);
          else
            store_chunk<TR, VEC>(pc, out);
        } else {
  #pragma unroll
          for (int e = 0; e < V; ++e) {
            if (grow[i] + e < m_end) {
              T o = alpha * v[e];
              if (read_c) o = fma_t(beta, pc[e], o);
              pc[e] = o;
            }
          }
        }
      }
      return;
    }

    if constexpr (KS > 1) {
      // Groups 1 .. KS-1 hand their partial sums to group 0 through LDS
      // (lane-linear, so each register index is one contiguous 256-byte row
      // per wave; one region per group); group 0 adds them in group order
      // and runs the epilogue alone.
      constexpr int NREG = RB * CB * TR::NACC;
      __syncthreads();                       // every wave is done with the ring
      T* const red = lds + wave_in * NREG * 64 + lane;
      constexpr int GSTRIDE = WGM * WGN * NREG * 64;   // elements per group's region
      if (kgrp > 0) {
        T* const mine = red + (kgrp - 1) * GSTRIDE;
  #pragma unroll
        for (int b = 0; b < RB; ++b)
  #pragma unroll
          for (int c = 0; c < CB; ++c)
  #pragma unroll
            for (int e = 0; e < TR::NACC; ++e) mine[((b * CB + c) * TR::NACC + e) * 64] = acc[b][c][e];
      }
      __syncthreads();
      if (kgrp == 0) {
  #pragma unroll
        for (int j = 0; j < KS - 1; ++j)
  #pragma unroll
          for (int b = 0; b < RB; ++b)
  #pragma unroll
            for (int c = 0; c < CB; ++c)
  #pragma unroll
              for (int e = 0; e < TR::NACC; ++e)
                acc[b][c][e] += red[j * GSTRIDE + ((b * CB + c) * TR::NACC + e) * 64];
      }
      // the epilogue's staging reuses this LDS: every read of it is done first
      __syncthreads();
      if (kgrp != 0) return;
    }

    // Destination: C, or for a stream-K piece its raw partial sums (alpha = 1,
    // beta = 0, all BM x BN elements, column-major with ld = BM) in workspace
    // slot `slot`.
    const bool to_ws = slot >= 0;
    T* const cbase = to_ws ? g.ws + (size_t)slot * (BM * BN) : g.C;
    const int ldc = to_ws ? BM : g.ldc;
    const T alpha = to_ws ? T(1) : g.alpha, beta = to_ws ? T(0) : g.beta;
    const bool read_c = beta != T(0);
    if constexpr (Cfg::STAGED_EPI) {
      // Staged through LDS so that global memory sees whole column segments.
      // Per column block c, each wave writes its MB columns x WM rows to a
      // private LDS region, then reads it back a 16-byte chunk per lane with
      // consecutive lanes on consecutive rows: a wave's store covers whole
      // columns (WM*sizeof(T) bytes each) instead of 16 bytes in each of 32
      // columns.  Chunk h of column j sits at chunk h ^ (j & 7) of the column's
      // WM/V chunks: the 8 lanes of a ds_write_b128 cycle (8 consecutive
      // columns, one chunk index) then hit 8 distinct bank groups, and each read
      // cycle (8-lane blocks b and b^3) covers 16 distinct groups of a 256-byte
      // line.  Only this wave touches its region, and a wave's LDS operations
      // complete in order, so no barrier is needed.
      const int m_end = to_ws ? BM : M, n_end = to_ws ? BN : N;   // extent in that frame
      const int row_base = (to_ws ? 0 : m0) + wrow, col_base = (to_ws ? 0 : n0) + wcol;
      constexpr int LDW = Cfg::EPI_LDW;            // staging column stride (elements)
      constexpr int CPC = Cfg::WM / V;             // chunks per wave-tile column
      constexpr int NCH = MB * CPC;                // chunks per column block
      static_assert(RUN % V == 0, "a run is whole 16-byte chunks");
      static_assert(NCH % 64 == 0, "whole chunks per lane");
      T* const stg = lds + wave_in * (MB * LDW);
      // A whole chunk of C (or of the workspace slot) at (gcol, grow) of this
      // frame.  Written through in the fp32 64 x 64 class (TileCfg::WT_C),
      // from the frame's first element with 32-bit byte offsets.  Measured
      // there on 1024^3 (workspace-free launches, back to back): -1.6 % with
      // beta = 0 and -1.4 % with beta = 0.5; at 896^3 and 1000^3 with
      // beta = 0.5 -9 % and -11 %, and -17 % at ldc 1280.  Ordinary stores
      // cost an L2 write-back of C at the kernel's end, and with beta != 0
      // at most leading dimensions a further ~3 us.  A run-time choice
      // between the two at each store measured slower than either.
      const int col0 = to_ws ? 0 : n0, row0 = to_ws ? 0 : m0;
      auto put_chunk = [&](const int gcol, const int grow, const chunk_t& out)
                           __attribute__((always_inline)) {
        if constexpr (Cfg::WT_C)
          store_chunk_wt<TR>(tile_rsrc(cbase + (size_t)col0 * ldc + row0),
                             ((gcol - col0) * ldc + (grow - row0)) * (int)sizeof(T), out);
        else
          store_chunk<TR, VEC>(cbase + (size_t)gcol * ldc + grow, out);
      };
      // With beta != 0 and the whole tile inside C, the old C of column block
      // c+1 is loaded as soon as block c is staged (its accumulators are free
      // then), so that its HBM latency passes while block c is stored; block
      // 0's loads go out before its staging.
      constexpr int NI = NCH / 64;                 // chunks per lane per column block
      const bool pre_c = read_c && !to_ws && full_mn;
      chunk_t cpre[2][NI];
      auto load_c_block = [&](int c, chunk_t (&dst)[NI]) {
  #pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int q = lane + 64 * i;
          const int col = q / CPC, rc = q % CPC;
          dst[i] = load_chunk_full<TR, VEC>(cbase + (size_t)(col_base + c * MB + col) * ldc +
                                            (row_base + rc * V));
        }
      };
      if constexpr (PF_C) {
        // the K loop was too short to load the old C: every chunk now
        static_assert(NI == Cfg::EPI_NI && NPF == CB * NI, "prefetch layout is the epilogue's");
        if (pre_c && !pf_done) {
  #pragma unroll
          for (int q = 0; q < NPF; ++q) cpf[q] = load_c_chunk(q);
        }
        if (pre_c && pf_done) {
  #pragma unroll
          for (int q = NPF - NPF_LATE; q < NPF; ++q) cpf[q] = load_c_chunk(q);   // not prefetched
        }
      } else {
        if (pre_c) load_c_block(0, cpre[0]);
      }
  #pragma unroll
      for (int c = 0; c < CB; ++c) {
  #pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
  #pragma unroll
          for (int run = 0; run < NRUN; ++run) {
            T* const pcol = stg + lrow * LDW;
            const int ch0 = (sb * MB * W + W * TR::irow(run, kslot)) / V;
  #pragma unroll
            for (int h = 0; h < RUN / V; ++h) {
              chunk_t v;
  #pragma unroll
              for (int e = 0; e < V; ++e) {
                const int o = h * V + e;
                v[e] = acc[sb * W + o % W][c][run * TR::RUN_R + o / W];
              }
              *reinterpret_cast<chunk_t*>(pcol + ((ch0 + h) ^ (lrow & 7)) * V) = v;
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the staging is written
        if (pre_c) {
          if constexpr (!PF_C) {
            if (c + 1 < CB) load_c_block(c + 1, cpre[(c + 1) & 1]);
          }
  #pragma unroll
          for (int i = 0; i < NI; ++i) {
            const int q = lane + 64 * i;
            const int col = q / CPC, rc = q % CPC;
            const chunk_t v =
                *reinterpret_cast<const chunk_t*>(stg + col * LDW + (rc ^ (col & 7)) * V);
            chunk_t cold;
            if constexpr (PF_C) cold = cpf[c * NI + i];
            else cold = cpre[c & 1][i];
            chunk_t out;
  #pragma unroll
            for (int e = 0; e < V; ++e) out[e] = fma_t(beta, cold[e], alpha * v[e]);
            put_chunk(col_base + c * MB + col, row_base + rc * V, out);
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the region is reused
          continue;
        }
  #pragma unroll
        for (int i = 0; i < NCH / 64; ++i) {
          const int q = lane + 64 * i;
          const int col = q / CPC, rc = q % CPC;
          const chunk_t v = *reinterpret_cast<const chunk_t*>(stg + col * LDW + (rc ^ (col & 7)) * V);
          const int gcol = col_base + c * MB + col, grow = row_base + rc * V;
          if (gcol < n_end) {
            T* pc = cbase + (size_t)gcol * ldc + grow;
            if (grow + V <= m_end) {
              chunk_t out;
              if (read_c) {
                const chunk_t cv = load_chunk_full<TR, VEC>(pc);
  #pragma unroll
                for (int e = 0; e < V; ++e) out[e] = fma_t(beta, cv[e], alpha * v[e]);
              } else {
  #pragma unroll
                for (int e = 0; e < V; ++e) out[e] = alpha * v[e];
              }
              put_chunk(gcol, grow, out);
            } else {
  #pragma unroll
              for (int e = 0; e < V; ++e) {
                if (grow + e < m_end) {
                  T o = alpha * v[e];
                  if (read_c) o = fma_t(beta, pc[e], o);
                  pc[e] = o;
                }
              }
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the region is reused
      }
    } else {
      // Direct stores from the accumulator registers: runs of RUN rows of a
      // column per lane, 16-byte stores where whole chunks (written through,
      // from the frame's first element, in the 64 x 64 class: TileCfg::WT_C).
      const bool full_out = to_ws || full_mn;
      const int row_off = to_ws ? 0 : m0, col_off = to_ws ? 0 : n0;
      constexpr bool VEC_C = (RUN % V == 0);   // whole 16-byte chunks per run
      // The old C of group (c, sb): NRUN runs of RUN rows of this lane's column.
      auto load_c_group = [&](int c, int sb, T (&cv)[NRUN][RUN]) {
        const T* pcol = cbase + (size_t)(col_off + wcol + c * MB + lrow) * ldc;
        const int row0 = row_off + wrow + sb * MB * W;
  #pragma unroll
        for (int run = 0; run < NRUN; ++run) {
          const T* pc = pcol + row0 + W * TR::irow(run, kslot);
          if constexpr (VEC_C) {
  #pragma unroll
            for (int h = 0; h < RUN / V; ++h) {
              chunk_t v = load_chunk_full<TR, VEC>(pc + h * V);
  #pragma unroll
              for (int e = 0; e < V; ++e) cv[run][h * V + e] = v[e];
            }
          } else {
  #pragma unroll
            for (int o = 0; o < RUN; ++o) cv[run][o] = pc[o];
          }
        }
      };
      if (read_c && full_mn && !to_ws) {
        // Whole tile inside C with beta != 0.
        auto put_group = [&](const int c, const int sb, const T (&cv)[NRUN][RUN])
                             __attribute__((always_inline)) {
          T* pcol = cbase + (size_t)(col_off + wcol + c * MB + lrow) * ldc;
          const int row0 = row_off + wrow + sb * MB * W;
  #pragma unroll
          for (int run = 0; run < NRUN; ++run) {
            T* pc = pcol + row0 + W * TR::irow(run, kslot);
            T out[RUN];
  #pragma unroll
            for (int o = 0; o < RUN; ++o)
              out[o] = fma_t(beta, cv[run][o],
                             alpha * acc[sb * W + o % W][c][run * TR::RUN_R + o / W]);
            if constexpr (VEC_C) {
  #pragma unroll
              for (int h = 0; h < RUN / V; ++h) {
                chunk_t v;
  #pragma unroll
                for (int e = 0; e < V; ++e) v[e] = out[h * V + e];
                if constexpr (Cfg::WT_C)
                  store_chunk_wt<TR>(tile_rsrc(cbase + (size_t)col_off * ldc + row_off),
                                     (int)((pc + h * V) - (cbase + (size_t)col_off * ldc + row_off)) *
                                         (int)sizeof(T),
                                     v);
                else
                  store_chunk<TR, VEC>(pc + h * V, v);
              }
            } else {
  #pragma unroll
              for (int o = 0; o < RUN; ++o) pc[o] = out[o];
            }
          }
        };
        constexpr int NG_EPI = CB * SB;
        if constexpr (PF_CT) {
          if (ct_done) {
            // loaded during the last K tiles
  #pragma unroll
            for (int gq = 0; gq < NG_EPI; ++gq) put_group(gq / SB, gq % SB, ct[gq]);
            return;
          }
        }
        // Otherwise the old C of the next group is loaded before this group's
        // multiply-adds and stores, so that one HBM latency is exposed per
        // tile instead of one per group.
        T cvb[2][NRUN][RUN];
        load_c_group(0, 0, cvb[0]);
  #pragma unroll
        for (int gq = 0; gq < NG_EPI; ++gq) {
          if (gq + 1 < NG_EPI) load_c_group((gq + 1) / SB, (gq + 1) % SB, cvb[(gq + 1) & 1]);
          put_group(gq / SB, gq % SB, cvb[gq & 1]);
        }
        return;
      }
  #pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int col = col_off + wcol + c * MB + lrow;
        T* pcol = cbase + (size_t)col * ldc;
  #pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const int row0 = row_off + wrow + sb * MB * W;
          if (full_out) {
            // Whole tile in range: issue every C load of this column block
            // first, then the multiply-adds and stores, so that the loads'
            // latency is paid once rather than once per run.
            T cv[NRUN][RUN];
            if (read_c) load_c_group(c, sb, cv);
  #pragma unroll
            for (int run = 0; run < NRUN; ++run) {
              T* pc = pcol + row0 + W * TR::irow(run, kslot);
              T out[RUN];
  #pragma unroll
              for (int o = 0; o < RUN; ++o) {
                out[o] = alpha * acc[sb * W + o % W][c][run * TR::RUN_R + o / W];
                if (read_c) out[o] = fma_t(beta, cv[run][o], out[o]);
              }
              if constexpr (VEC_C) {
  #pragma unroll
                for (int h = 0; h < RUN / V; ++h) {
                  chunk_t v;
  #pragma unroll
                  for (int e = 0; e < V; ++e) v[e] = out[h * V + e];
                  if constexpr (Cfg::WT_C)
                    store_chunk_wt<TR>(tile_rsrc(cbase + (size_t)col_off * ldc + row_off),
                                       (int)((pc + h * V) - (cbase + (size_t)col_off * ldc + row_off)) *
                                           (int)sizeof(T),
                                       v);
                  else
                    store_chunk<TR, VEC>(pc + h * V, v);
                }
              } else {
  #pragma unroll
                for (int o = 0; o < RUN; ++o) pc[o] = out[o];
              }
            }
          } else if (col < N) {
            // Edge tile: element-wise bounds checks.
  #pragma unroll
            for (int run = 0; run < NRUN; ++run) {
              const int row = row0 + W * TR::irow(run, kslot);
              T* pc = pcol + row;
  #pragma unroll
              for (int o = 0; o < RUN; ++o) {
                if (row + o < M) {
                  T v = alpha * acc[sb * W + o % W][c][run * TR::RUN_R + o / W];
                  if (read_c) v = fma_t(beta, pc[o], v);
                  pc[o] = v;
                }
              }
            }
          }
        }
      }
    }
  };  // tile_piece

  if constexpr (!SKP) {
    tile_piece(xcd_remap(blockIdx.x, g.full_tiles), 0, nk_all, -1);
  } else {
    // With K groups, the groups other than 0 leave a piece after the
    // hand-over (every group has passed the same barriers) while group 0
    // runs the epilogue, which has none; all meet again at the barrier below.
    for (int pc = 0; pc < npieces; ++pc) {
      int t_lin, kb = 0, ke = nk_all, slot = -1;
      if (!sk_wg) {
        t_lin = xcd_remap(blockIdx.x, g.full_tiles);
      } else {
        // the previous piece's epilogue has finished with the LDS
        if (pc > 0) __syncthreads();
        const int r = sk_r0 + pc;
        const long long first = (long long)r * nk_all;
        t_lin = g.full_tiles + r;
        if (pc == 0) kb = (int)(sk_b0 - first);
        if (sk_b1 - first < nk_all) ke = (int)(sk_b1 - first);
        slot = 2 * w_sk + pc;
      }
      // one call site: the body is inlined once
      tile_piece(t_lin, kb, ke, slot);
    }
  }
}

// Fix-up of the stream-K tiles: C = alpha * (sum of the pieces' partial
// sums, in K order) + beta * C for every element of the remaining tiles that
// lies inside C.  Tile r's pieces come from the stream-K workgroups whose
// iteration ranges [b(w), b(w+1)), b(w) = floor(w*I/P), meet [r*nk,
// (r+1)*nk): workgroup w's piece is its slot 2w if its range starts in tile
// r, 2w + 1 if it started in tile r - 1.  One thread per element; block y =
// remaining tile.  The walk over w is the same for the whole block and
// steps b(w) by I/P with a remainder, without a division per step.
template <typename T>
__global__ void __launch_bounds__(256) sk_fixup_kernel(GemmArgs<T> g, int bm, int bn, int bk) {
  const int r = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;   // element of the tile, ld = bm
  if (e >= bm * bn) return;
  int tm, tn;
  raster(g.full_tiles + r, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
  const int i = tm * bm + e % bm, j = tn * bn + e / bm;
  if (i >= g.M || j >= g.N) return;
  const long long nk = (g.K + bk - 1) / bk;
  const long long rest = (long long)g.tiles_m * g.tiles_n - g.full_tiles;
  const long long iters = rest * nk, P = g.sk_wgs;
  const long long lo = (long long)r * nk, hi = lo + nk;
  const long long dq = iters / P, dr = iters % P;
  // w with b(w) <= lo, then b(w) = q and (w*I) mod P = rm
  long long w = (lo * P) / iters;
  long long q = (w * iters) / P, rm = (w * iters) % P;
  // b(w+1) from b(w)
  long long q1 = q + dq, rm1 = rm + dr;
  if (rm1 >= P) {
    ++q1;
    rm1 -= P;
  }
  // first workgroup whose range ends past lo
  while (q1 <= lo) {
    ++w;
    q = q1;
    rm = rm1;
    q1 = q + dq;
    rm1 = rm + dr;
    if (rm1 >= P) {
      ++q1;
      rm1 -= P;
    }
  }
  const size_t slot = (size_t)bm * bn;
  T sum = T(0);
  for (; w < P && q < hi; ++w) {
    sum += g.ws[(size_t)(2 * w + (q >= lo ? 0 : 1)) * slot + e];
    q += dq;
    rm += dr;
    if (rm >= P) {
      ++q;
      rm -= P;
    }
  }
  T* pc = g.C + (size_t)j * g.ldc + i;
  T v = g.alpha * sum;
  if (g.beta != T(0)) v = fma_t(g.beta, *pc, v);
  *pc = v;
}

// The strip of rows below the tile rows as a kernel of its own (for the
// tile classes whose workgroups leave no room beside them).  g.M is the
// whole height; rows [i0, g.M) form the strip.
constexpr int kStripThreads = 512, kStripLdsElems = 8192;
template <typename T>
constexpr int strip_kernel_scmax() {
  return sizeof(T) == 4 ? 8 : 4;
}
template <typename T>
constexpr int strip_kernel_acc() {
  return sizeof(T) == 4 ? 32 : 16;
}

template <typename T>
__global__ void __launch_bounds__(kStripThreads) strip_rows_kernel(GemmArgs<T> g, int i0) {
  constexpr int LDSE = kStripLdsElems;
  __shared__ __attribute__((aligned(16))) T lds[LDSE];
  strip_rows_wg<T, kStripThreads, strip_kernel_scmax<T>(), strip_kernel_acc<T>(), LDSE>(
      g, i0, g.M - i0, blockIdx.x, lds);
}

// C <- beta*C on the m x n block (the k == 0 / alpha == 0 path); beta == 0
// writes zeros without reading C.
template <typename T>
__global__ void __launch_bounds__(256) scale_kernel(int M, int N, T beta, T* C, int ldc) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M) return;
  for (int j = blockIdx.y; j < N; j += gridDim.y) {
    T* p = C + (size_t)j * ldc + i;
    *p = (beta == T(0)) ? T(0) : beta * *p;
  }
}

}  // namespace pgemm
