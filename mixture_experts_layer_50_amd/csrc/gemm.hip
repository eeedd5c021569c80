// Grouped GEMM kernels of the MoE layer for gfx950.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (fp32 accumulation) on LDS-staged
// 64-deep K slices in two LDS buffers, with further slices in flight in
// registers.  Operands stored k-contiguous sit in LDS the same way (16-byte
// chunks XOR-swizzled by row); operands stored n-contiguous (weights [K][N],
// activations read transposed) are copied as is and read back with the gfx950
// LDS transpose read.  Tiles are ordered so that consecutive tiles land on the
// same XCD (its own L2) and tiles that share an A row block or a weight column
// block run together (GROUP_M order).  Four kernel forms:
//  * gemm_bf16_kernel: one workgroup per tile;
//  * gemm_bf16_persistent_kernel: one workgroup per CU running a list of
//    tiles with the K-slice pipeline running on across tile boundaries;
//  * gemm_bf16_dma_kernel: persistent and warp-specialised (producer waves
//    copy K slices straight into LDS, compute waves multiply and store), for
//    plain-store epilogues with much output per unit of work (the weight
//    gradients, the down projection);
//  * gemm_bf16_ws_kernel: the same with register-staged producers (the down
//    projection with the combine fused into its epilogue).
// The gather roles read the rows of their A operand through a table of row
// numbers (the permuted rows Xp read from x: the dispatch copy folded into
// the GEMM's operand loads, page "Accelerating Transformers fine-tuning with
// NVIDIA NeMo AutoModel", section 加速来源, DeepEP item).
//
// fp32 path: a plain fp32 kernel (one output per thread, fp32 FMA) used for
// fp32 layers, which are small parity workloads.
#include <algorithm>
#include <utility>

#include "gemm.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;  // K extent of one LDS stage: 8 chunks of 8 bf16
constexpr int NXCD = 8;

// Physical 16-byte chunk of logical chunk c in LDS row r (conflict-free for
// 8 or 16 consecutive rows reading the same logical chunk).
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// Hardware dispatches workgroup ids round-robin over the 8 XCDs.  Give each
// XCD a contiguous range of the `count` real tiles instead.
__device__ __forceinline__ int remap_xcd(int pid, int count) {
  int xcd = pid % NXCD, idx = pid / NXCD;
  int per = count / NXCD, rem = count % NXCD;
  return xcd * per + min(xcd, rem) + idx;
}

// Linear tile id -> (m tile, n tile), GM m tiles at a time over all n tiles.
#ifndef MOE_GROUP_M
#define MOE_GROUP_M 4
#endif
__device__ __forceinline__ void group_order(int L, int mt_count, int nt_count, int& mt, int& nt) {
  constexpr int GM = MOE_GROUP_M;
  int per_group = GM * nt_count;
  int g = L / per_group;
  int first = g * GM;
  int gsize = min(mt_count - first, GM);
  int r = L - g * per_group;
  mt = first + r % gsize;
  nt = r / gsize;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ---------------------------------------------------------------------------
// LDS tile layouts.  One K slice is 64 deep.
//  k-contiguous operand ("KC"): [ROWS][64] bf16; 16-byte chunk c of row r sits
//    at chunk swz(r, c).  A lane reads its 8 k values with one 16-byte read.
//  k-major operand ("KN", stored n-contiguous in memory, e.g. a weight matrix
//    [K][N]): copied as is into [64][COLS]; chunk c of row k sits at
//    kn_swz(k, c).  A lane gathers 8 k values of one column with two
//    ds_read_b64_tr_b16 reads: in each group of 16 lanes, lane 4r+q addresses
//    row r, columns 4q..4q+3, and lane i receives column i of rows 0..3.
// ---------------------------------------------------------------------------
template <int COLS>
__device__ __forceinline__ int kn_swz(int k, int c) {
  return c ^ (((k & 3) << 2) & (COLS / 8 - 1));
}

// Buffer loads: the hardware returns zeros for a byte offset past num_records,
// so masked lanes get offset OOB and no lane branches around a load.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int OOB = (int)0x80000000u;

// A buffer descriptor over `nrec` bytes from `base` (the hardware range check
// covers the vector offset; loads at or past nrec return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, int nrec) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return make_rsrc_n(base, 0x7fffffff);
}

// CPOL: cache-policy bits of the load (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
template <int CPOL>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL));
}

// The group offsets, the tile table and the gather rows are read-only for the GEMM kernels;
// reading them through the constant address space with a uniform index makes
// them scalar loads, which do not wait behind the vector loads in flight.
typedef __attribute__((address_space(4))) const int32_t cint32_t;
__device__ __forceinline__ int ld_table(const int32_t* tab, int i) { return ((cint32_t*)tab)[i]; }

// Loader of a KC tile: row r of the tile is src[(row0 + r) * ld + k], rows
// r >= row_hi - row0 read as zeros.  With TWO, k < ksplit comes from s0 and
// k >= ksplit from s1 at k - ksplit (ksplit is a multiple of 64, so one K
// slice never straddles it).  The per-lane address state is kept once; the
// loaded data lives in a separate register array per pipeline stage.
//
// GATHER: tile row r is row rows[row0 + r] of the source (the rows of Xp
// read from x through the token table); the row numbers are loaded once per
// tile.  rows == NULL: row row0 + r, addressed from the tile's first row as
// without GATHER (the byte offsets stay within one tile).
template <int ROWS, bool TWO, int NT, int CPOL, bool GATHER, bool FULLK>
struct LoaderKC {
  static_assert(!(GATHER && TWO), "a gathered operand has one source");
  static constexpr int CH = ROWS * 8;
  static constexpr int NR = (CH + NT - 1) / NT;
  struct Data { uint4 r[NR]; };
  int voff[NR];
  __amdgpu_buffer_rsrc_t rs0, rs1;
  const bf16_t *p0, *p1;  // FULLK: the sources at the tile's first row
  int ksplit, k_lo, k_hi;
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t* s1, int64_t ld, int row0,
                                       int row_hi, int k_lo_, int k_hi_, int ksplit_, int tid,
                                       const int32_t* rows) {
    p0 = GATHER && rows ? s0 : s0 + (int64_t)row0 * ld;
    p1 = TWO ? s1 + (int64_t)row0 * ld : p0;
    rs0 = make_rsrc(p0);
    rs1 = make_rsrc(p1);
    ksplit = ksplit_;
    k_lo = k_lo_;
    k_hi = k_hi_;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      int q = tid + NT * i;
      int row = q >> 3;
      bool ok = (CH % NT == 0 || q < CH) && row0 + row < row_hi;
      if (GATHER && rows) row = ok ? rows[row0 + row] : 0;
      voff[i] = ok ? (int)(((int64_t)row * ld + (q & 7) * 8) * 2) : OOB;
    }
  }
  // K slice starting at k_lo + kofs; load_part<J, NJ> sends the loads i
  // with i mod NJ == J only (a slice in NJ parts).  FULLK (K a multiple of
  // 64): a slice lies wholly inside K or wholly past it, and one past it
  // gets an empty descriptor, so each load takes its precomputed offset as
  // is (a per-load select would write a temporary right before the load,
  // which the compiler then orders behind every load in flight).
  template <int J, int NJ>
  __device__ __forceinline__ void load_part(Data& d, int kofs, int tid) const {
    int k0 = k_lo + kofs;
    int lim = k_hi - k0;
    if constexpr (FULLK) {
      const bf16_t* b = p0;
      if (TWO && k0 >= ksplit) { b = p1; k0 -= ksplit; lim = k_hi - ksplit - k0; }
      const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(b, lim > 0 ? 0x7fffffff : 0);
#pragma unroll
      for (int i = J; i < NR; i += NJ) d.r[i] = buf_load16<CPOL>(rs, voff[i], k0 * 2);
    } else {
      __amdgpu_buffer_rsrc_t rs = rs0;
      if (TWO && k0 >= ksplit) { rs = rs1; k0 -= ksplit; lim = k_hi - ksplit - k0; }
#pragma unroll
      for (int i = J; i < NR; i += NJ) {
        const int kc = ((tid + NT * i) & 7) * 8;
        d.r[i] = buf_load16<CPOL>(rs, kc < lim ? voff[i] : OOB, k0 * 2);
      }
    }
  }
  __device__ __forceinline__ void load(Data& d, int kofs, int tid) const { load_part<0, 1>(d, kofs, tid); }
  __device__ __forceinline__ static void store(const Data& d, bf16_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      int q = tid + NT * i;
      if (CH % NT == 0 || q < CH) {
        int row = q >> 3, c = q & 7;
        *reinterpret_cast<uint4*>(lds + row * BK + swz(row, c) * 8) = d.r[i];
      }
    }
  }
};

// Loader of a KN tile: element (k, c) of the tile is src[(k_lo + kofs + k) * ld
// + col0 + c]; rows at or past k_hi and columns at or past col_hi read as
// zeros.  HALF: tile columns [0, COLS/2) come from s0 at col0 + c, columns
// [COLS/2, COLS) from s1 at col0 + c - COLS/2 (the gate | up halves); each
// load instruction reads one half only, so its buffer descriptor is uniform.
//
// Rows past k_hi: by default each K slice gets its own descriptor whose
// record count ends at the last valid row, so a load takes its precomputed
// offset as is.  SEL masks them with a per-load select instead (a temporary
// written right before the load; the compiler then orders it behind loads
// in flight, which measured faster where the A operand is gathered).
//
// GATHER: row k of the K range is row rows[k] of the source.  The lanes
// of one wave cover 64 / CPR consecutive rows per load, so each wave reads
// its row numbers with scalar loads, one K slice ahead of the data loads
// (scalar loads retire through their own counter, so waiting for them never
// waits for data loads in flight).
template <int COLS, bool HALF, int NT, int CPOL, bool GATHER, bool SEL>
struct LoaderKN {
  static constexpr int CPR = HALF ? COLS / 16 : COLS / 8;  // chunks per row and source
  static constexpr int CH = BK * CPR;                        // chunks per source
  static constexpr int NS = (CH + NT - 1) / NT;              // loads per source
  static constexpr int NR = HALF ? 2 * NS : NS;
  static constexpr int RW = GATHER ? 64 / CPR : 1;           // rows per wave and load (GATHER)
  static_assert(!GATHER || (!HALF && 64 % CPR == 0 && NT % 64 == 0 && CH % NT == 0),
                "gathered rows: whole rows per wave");
  struct Data { uint4 r[NR]; };
  int voff[NS];  // byte offset of the lane's chunk from the slice's first row (OOB: masked column)
  __amdgpu_buffer_rsrc_t rs0, rs1;  // GATHER, SEL
  const bf16_t *p0, *p1;            // the sources at (k_lo, col0)
  int64_t ld;
  int k_lo, k_hi;
  const int32_t* rows;
  int wrow;         // GATHER: the wave's first row of load 0
  int nxt[NS][RW];  // GATHER: row numbers of the next slice (wave-uniform)
  __device__ __forceinline__ void prefetch(int kofs) {
    // the pointer is the same in every lane; say so, or the loads stay vector loads
    const uint64_t a = (uint64_t)rows;
    const int32_t* tab = (const int32_t*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                                          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a));
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < RW; ++j)
        nxt[i][j] = ld_table(tab, min(k_lo + kofs + wrow + i * (NT / CPR) + j, k_hi - 1));
  }
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t* s1, int64_t ld_, int col0,
                                       int col_hi, int k_lo_, int k_hi_, int, int tid,
                                       const int32_t* rows_) {
    ld = ld_;
    k_lo = k_lo_;
    k_hi = k_hi_;
    p0 = s0 + (int64_t)k_lo * ld + col0;
    p1 = (HALF ? s1 : s0) + (int64_t)k_lo * ld + col0;
    rs0 = make_rsrc(GATHER ? s0 + col0 : p0);
    rs1 = make_rsrc(p1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      int q = tid + NT * i;
      int col = (q % CPR) * 8;
      bool ok = (CH % NT == 0 || q < CH) && col0 + col < col_hi;
      voff[i] = ok ? (int)(((GATHER ? 0 : (int64_t)(q / CPR) * ld) + col) * 2) : OOB;
    }
    if constexpr (GATHER) {
      rows = rows_;
      wrow = __builtin_amdgcn_readfirstlane((tid >> 6) * (64 / CPR));
      if (k_hi > k_lo) prefetch(0);  // an empty K range has no row numbers
    }
  }
  // K slice starting at k_lo + kofs
  __device__ __forceinline__ void load(Data& d, int kofs, int tid) {
    if constexpr (GATHER) {
      const int lim = k_hi - k_lo - kofs;
      const int sub = (tid & 63) / CPR;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        int r = nxt[i][0];
#pragma unroll
        for (int j = 1; j < RW; ++j) r = sub == j ? nxt[i][j] : r;
        const bool ok = (tid + NT * i) / CPR < lim && voff[i] != OOB;
        d.r[i] = buf_load16<CPOL>(rs0, ok ? (int)(r * ld * 2) + voff[i] : OOB, 0);
      }
      if (kofs + BK < k_hi - k_lo) prefetch(kofs + BK);
      return;
    }
    load_part<0, 1>(d, kofs, tid);
  }
  // the loads i with i mod NJ == J only (not for GATHER)
  template <int J, int NJ>
  __device__ __forceinline__ void load_part(Data& d, int kofs, int tid) const {
    static_assert(!GATHER || NJ == 1, "gathered rows load whole slices");
    const int lim = k_hi - k_lo - kofs;
    if constexpr (SEL) {
      const int soff = (int)((int64_t)kofs * ld * 2);
#pragma unroll
      for (int i = J; i < NS; i += NJ) {
        const int v = (tid + NT * i) / CPR < lim ? voff[i] : OOB;
        d.r[i] = buf_load16<CPOL>(rs0, v, soff);
        if (HALF) d.r[NS + i] = buf_load16<CPOL>(rs1, v, soff);
      }
    } else {
      const int nrec = lim <= 0 ? 0 : lim >= BK ? 0x7fffffff : (int)((int64_t)lim * ld * 2);
      const __amdgpu_buffer_rsrc_t r0 = make_rsrc_n(p0 + (int64_t)kofs * ld, nrec);
      const __amdgpu_buffer_rsrc_t r1 = make_rsrc_n(p1 + (int64_t)kofs * ld, nrec);
#pragma unroll
      for (int i = J; i < NS; i += NJ) {
        d.r[i] = buf_load16<CPOL>(r0, voff[i], 0);
        if (HALF) d.r[NS + i] = buf_load16<CPOL>(r1, voff[i], 0);
      }
    }
  }
  __device__ __forceinline__ static void store(const Data& d, bf16_t* lds, int tid) {
#pragma unroll
    for (int h = 0; h < (HALF ? 2 : 1); ++h) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        int q = tid + NT * i;
        if (CH % NT == 0 || q < CH) {
          int k = q / CPR, c = q % CPR + h * CPR;
          *reinterpret_cast<uint4*>(lds + k * COLS + kn_swz<COLS>(k, c) * 8) = d.r[h * NS + i];
        }
      }
    }
  }
};

// FULLK: K is a multiple of 64 (KC loaders); SEL: per-load row selects (KN)
template <bool KC, int ROWS, bool TWO, int NT, int CPOL, bool GATHER, bool FULLK, bool SEL>
struct PickLoader;
template <int ROWS, bool TWO, int NT, int CPOL, bool GATHER, bool FULLK, bool SEL>
struct PickLoader<true, ROWS, TWO, NT, CPOL, GATHER, FULLK, SEL> {
  typedef LoaderKC<ROWS, TWO, NT, CPOL, GATHER, FULLK> type;
};
template <int ROWS, bool TWO, int NT, int CPOL, bool GATHER, bool FULLK, bool SEL>
struct PickLoader<false, ROWS, TWO, NT, CPOL, GATHER, FULLK, SEL> {
  typedef LoaderKN<ROWS, TWO, NT, CPOL, GATHER, SEL> type;
};

// ---------------------------------------------------------------------------
// Loaders that copy a K slice from memory straight into LDS (gfx950 16-byte
// buffer loads with the LDS as destination: lane l of a load writes bytes
// [16 l, 16 l + 16) from the load's LDS address on, and a lane past the
// buffer's range writes zeros).  Load i of producer wave w fills the 64
// consecutive physical chunks from 64 w + NT i on, so each lane loads the
// logical chunk that the slice's layout puts at its physical slot (the
// swizzles are XORs of the chunk index, their own inverses): the LDS layout
// is the register-staged loaders' exactly.  K must be a multiple of 64 for
// the k-contiguous form; the k-major form reads rows past the K range as
// zeros through the buffer's range (or masked offsets when gathered).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

template <int CPOL>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, bf16_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, CPOL);
}

template <int ROWS, int NT, int CPOL>
struct DmaKC {
  static constexpr int CH = ROWS * 8;
  static constexpr int NR = CH / NT;
  static constexpr int NLOAD = NR;  // loads per producer thread and slice
  static_assert(CH % NT == 0, "whole loads per producer thread");
  int voff[NR];
  const bf16_t* p0;
  int k_lo, k_hi;
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t*, int64_t ld, int row0,
                                       int row_hi, int k_lo_, int k_hi_, int, int tid,
                                       const int32_t*) {
    p0 = s0 + (int64_t)row0 * ld;
    k_lo = k_lo_;
    k_hi = k_hi_;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = tid + NT * i, row = q >> 3;
      const int c = (q & 7) ^ (row & 7) ^ ((row >> 3) & 1);  // swz(row, .) inverted
      voff[i] = row0 + row < row_hi ? (int)(((int64_t)row * ld + c * 8) * 2) : OOB;
    }
  }
  // the slice starting at k_lo + kofs into `lds` (this operand's tile)
  __device__ __forceinline__ void issue(bf16_t* lds, int kofs, int tid) const {
    const int k0 = k_lo + kofs;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_n(p0, k_hi - k0 > 0 ? 0x7fffffff : 0);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int i = 0; i < NR; ++i) dma16<CPOL>(rs, lds + (64 * w + NT * i) * 8, voff[i], k0 * 2);
  }
};

template <int COLS, int NT, int CPOL, bool GATHER>
struct DmaKN {
  static constexpr int CPR = COLS / 8;  // chunks per row
  static constexpr int CH = BK * CPR;
  static constexpr int NS = CH / NT;
  static constexpr int RW = GATHER ? 64 / CPR : 1;  // rows per wave and load (GATHER)
  static constexpr int NLOAD = NS;                   // loads per producer thread and slice
  static_assert(CH % NT == 0 && (!GATHER || (64 % CPR == 0 && NT % 64 == 0)), "load shape");
  int voff[NS];  // byte offset of the lane's chunk (OOB: masked column)
  __amdgpu_buffer_rsrc_t rs0;  // GATHER
  const bf16_t* p0;            // the source at (k_lo, col0)
  int64_t ld;
  int k_lo, k_hi;
  const int32_t* rows;
  int wrow;
  int nxt[NS][RW];
  __device__ __forceinline__ void prefetch(int kofs) {
    const uint64_t a = (uint64_t)rows;
    const int32_t* tab = (const int32_t*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                                          (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a));
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < RW; ++j)
        nxt[i][j] = ld_table(tab, min(k_lo + kofs + wrow + i * (NT / CPR) + j, k_hi - 1));
  }
  __device__ __forceinline__ void init(const bf16_t* s0, const bf16_t*, int64_t ld_, int col0,
                                       int col_hi, int k_lo_, int k_hi_, int, int tid,
                                       const int32_t* rows_) {
    ld = ld_;
    k_lo = k_lo_;
    k_hi = k_hi_;
    p0 = s0 + (int64_t)k_lo * ld + col0;
    rs0 = make_rsrc(s0 + col0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int q = tid + NT * i, k = q / CPR;
      const int col = ((q % CPR) ^ (((k & 3) << 2) & (CPR - 1))) * 8;  // kn_swz(k, .) inverted
      voff[i] = col0 + col < col_hi ? (int)(((GATHER ? 0 : (int64_t)k * ld) + col) * 2) : OOB;
    }
    if constexpr (GATHER) {
      rows = rows_;
      wrow = __builtin_amdgcn_readfirstlane((tid >> 6) * (64 / CPR));
      if (k_hi > k_lo) prefetch(0);
    }
  }
  __device__ __forceinline__ void issue(bf16_t* lds, int kofs, int tid) {
    const int lim = k_hi - k_lo - kofs;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if constexpr (GATHER) {
      const int sub = (tid & 63) / CPR;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        int r = nxt[i][0];
#pragma unroll
        for (int j = 1; j < RW; ++j) r = sub == j ? nxt[i][j] : r;
        const bool ok = (tid + NT * i) / CPR < lim && voff[i] != OOB;
        dma16<CPOL>(rs0, lds + (64 * w + NT * i) * 8, ok ? (int)(r * ld * 2) + voff[i] : OOB, 0);
      }
      if (kofs + BK < k_hi - k_lo) prefetch(kofs + BK);
    } else {
      const int nrec = lim <= 0 ? 0 : lim >= BK ? 0x7fffffff : (int)((int64_t)lim * ld * 2);
      const __amdgpu_buffer_rsrc_t r0 = make_rsrc_n(p0 + (int64_t)kofs * ld, nrec);
#pragma unroll
      for (int i = 0; i < NS; ++i) dma16<CPOL>(r0, lds + (64 * w + NT * i) * 8, voff[i], 0);
    }
  }
};

// MFMA operand fragment (32 rows x 16 k): lane l holds row base + (l & 31),
// k = 16 ks + 8 (l >> 5) + 0..7.
__device__ __forceinline__ bf16x8 frag_kc(const bf16_t* lds, int base, int ks, int lane) {
  const int row = base + (lane & 31);
  const int c = ks * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(lds + row * BK + swz(row, c) * 8);
}

template <int COLS>
__device__ __forceinline__ bf16x8 frag_kn(const bf16_t* lds, int base, int ks, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int col = base + ((g & 1) << 4) + ((j & 3) << 2);
  const int k = ks * 16 + ((g >> 1) << 3) + (j >> 2);
  const int off = k * COLS + kn_swz<COLS>(k, col >> 3) * 8 + (col & 7);  // k+4: same swizzle
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off + 4 * COLS));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Tiles.  Tile ids run over (expert for G_KROWS) x m tiles x n tiles; for
// G_MROWS the m tiles come from the device-built tile table.
// ---------------------------------------------------------------------------
struct TileDesc {
  int e;           // local expert (0 for G_DENSE)
  int m_lo, m_hi;  // output rows [m_lo, m_hi)
  int n0;          // first output column (gate|up: first column of each half)
  int k_lo, k_hi;  // K range
};


template <int GMD>
__device__ __forceinline__ int tile_count(const GemmParams& p) {
  const int mt_count = (GMD == G_MROWS) ? ld_table(p.tiles, 0) : p.m_tiles;
  const int per_group = mt_count * p.n_tiles;
  return (GMD == G_KROWS) ? per_group * p.groups : per_group;
}

// The tile id is the same in every lane; the integer divisions below run on
// the vector unit, so the indices are moved back to scalar registers before
// they address the tables.
template <int BM, int BN, int GMD, int B2>
__device__ __forceinline__ TileDesc tile_desc(const GemmParams& p, int L) {
  TileDesc t;
  const int mt_count = (GMD == G_MROWS) ? ld_table(p.tiles, 0) : p.m_tiles;
  t.e = 0;
  if (GMD == G_KROWS) {
    const int per_group = mt_count * p.n_tiles;
    t.e = __builtin_amdgcn_readfirstlane(L / per_group);
    L -= t.e * per_group;
  }
  int mt, nt;
  group_order(L, mt_count, p.n_tiles, mt, nt);
  mt = __builtin_amdgcn_readfirstlane(mt);
  nt = __builtin_amdgcn_readfirstlane(nt);
  if (GMD == G_MROWS) {
    t.e = ld_table(p.tiles, 1 + 2 * mt);
    t.m_lo = ld_table(p.tiles, 2 + 2 * mt);
    t.m_hi = min(t.m_lo + BM, ld_table(p.off, t.e + 1));
    t.k_lo = 0;
    t.k_hi = p.K;
  } else {
    t.m_lo = mt * BM;
    t.m_hi = min(t.m_lo + BM, p.M);
    if (GMD == G_KROWS && p.off) {
      t.k_lo = ld_table(p.off, t.e);
      t.k_hi = ld_table(p.off, t.e + 1);
      if (p.k_strip && ld_table(p.kcost, t.e + 1) == ld_table(p.kcost, t.e)) {  // the strip kernel's
        t.k_hi = t.k_lo;
        t.m_hi = t.m_lo;
      }
    }
    else if (GMD == G_KROWS && p.k_chunk > 0) {
      t.k_lo = min(p.K, t.e * p.k_chunk);
      t.k_hi = min(p.K, t.k_lo + p.k_chunk);
    } else { t.k_lo = 0; t.k_hi = p.K; }
  }
  t.n0 = nt * ((B2 == B2_NHALF) ? BN / 2 : BN);
  return t;
}

// The contiguous range [x_lo, x_lo + x_n) of tile ids a persistent kernel's
// XCD takes.  Tiles of the row-grouped and dense GEMMs cost the same, so the
// XCDs get equal counts.  Weight-gradient tiles cost their expert's K slices
// (plus a fixed part for the epilogue), which differ widely under natural
// routing: there the split is by cost, so that no XCD is left with the
// largest experts.
template <int GMD>
__device__ __forceinline__ void xcd_tile_range(const GemmParams& p, int count, int xcd, int& x_lo,
                                               int& x_n) {
  if (GMD != G_KROWS || p.kcost == nullptr) {
    const int per = count / NXCD, rem = count % NXCD;
    x_lo = xcd * per + min(xcd, rem);
    x_n = per + (xcd < rem ? 1 : 0);
    return;
  }
  const int per_group = count / p.groups;  // tiles per expert, all of the same cost
  const int64_t total = (int64_t)ld_table(p.kcost, p.groups) * per_group;
  // first tile whose cost prefix reaches c
  auto first_at = [&](int64_t c) -> int {
    if (c <= 0) return 0;
    if (c >= total) return count;
    int lo = 0, hi = p.groups - 1;  // last expert whose tiles start below c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)ld_table(p.kcost, mid) * per_group < c) lo = mid;
      else hi = mid - 1;
    }
    const int64_t before = (int64_t)ld_table(p.kcost, lo) * per_group;
    const int tc = ld_table(p.kcost, lo + 1) - ld_table(p.kcost, lo);
    return lo * per_group + (int)min<int64_t>(per_group, (c - before + tc - 1) / tc);
  };
  x_lo = first_at(total * xcd / NXCD);
  x_n = first_at(total * (xcd + 1) / NXCD) - x_lo;
}

#ifndef MOE_WEIGHT_CPOL
#define MOE_WEIGHT_CPOL 2
#endif
// Cache policy of the weight-gradient result stores (2 = nt).
#ifndef MOE_OUT_CPOL
#define MOE_OUT_CPOL 2
#endif

// Loader types of a GEMM.  The expert weights (B of the row-grouped GEMMs)
// stream through once and are loaded non-temporal; the activation rows (A)
// are re-read by every column tile of the expert and stay cached.
// The gather roles read the rows of A through a_rows.
constexpr bool gathers_a(int role) {
  return role == R_GATEUP_FWD_GATHER || role == R_GATEUP_WGRAD_GATHER || role == R_DOWN_DGRAD_GATHER;
}
// Roles whose k-contiguous operands have K a multiple of 64 (d or I, which
// the entry points require to be); the router's input gradient runs over the
// E expert logits instead.
constexpr bool full_k(int role) { return role != R_ROUTE_DX; }

template <int BM, int BN, int NT, int AM, int BMD, int GMD, int B2, bool AG, bool FK>
struct Loaders {
  static constexpr int BPOL = GMD == G_MROWS ? MOE_WEIGHT_CPOL : 0;
  // next to a gathered A operand, B keeps per-load selects (measured faster)
  typedef typename PickLoader<AM == A_KC, BM, false, NT, 0, AG, FK, AG>::type LA;
  typedef typename PickLoader<BMD == B_KC, BN, B2 != B2_NONE, NT, BPOL, false, FK, AG>::type LB;
};

// The copy-to-LDS loaders of a GEMM (one B source; cache policies as above).
template <int BM, int BN, int NT, int AM, int BMD, int GMD, bool AG>
struct DmaLoaders {
  static constexpr int BPOL = GMD == G_MROWS ? MOE_WEIGHT_CPOL : 0;
  template <bool KC, int N_, int CP, bool G_> struct Pick { typedef DmaKN<N_, NT, CP, G_> type; };
  template <int N_, int CP, bool G_> struct Pick<true, N_, CP, G_> { typedef DmaKC<N_, NT, CP> type; };
  typedef typename Pick<AM == A_KC, BM, 0, AG>::type LA;
  typedef typename Pick<BMD == B_KC, BN, BPOL, false>::type LB;
  static constexpr int LOADS = LA::NLOAD + LB::NLOAD;  // per producer thread and slice
};

// R_DOWN_DGRAD_GATHER reads the materialised dYp (a_alt) when the weight
// gradients' tile kernels have work (see GemmParams::a_alt).
__device__ __forceinline__ bool reads_alt(const GemmParams& p) {
  return p.a_alt != nullptr && ld_table(p.kcost, p.groups) != 0;
}

template <int GMD, int B2, typename LA, typename LB>
__device__ __forceinline__ void init_loaders(const GemmParams& p, const TileDesc& t, LA& la, LB& lb,
                                             int tid) {
  // (a select of the two pointer values: a select of the two kernel
  // arguments as lvalues put them in scratch memory)
  const bool alt = reads_alt(p);
  const void* a_main = p.A;
  const void* a_dyp = p.a_alt;
  const bf16_t* A = static_cast<const bf16_t*>(alt ? a_dyp : a_main);
  const bf16_t* B0 = static_cast<const bf16_t*>(p.B0);
  const bf16_t* B1 = static_cast<const bf16_t*>(p.B1);
  if (GMD == G_MROWS) {
    B0 += (int64_t)t.e * p.b_estride;
    if (B2 != B2_NONE) B1 += (int64_t)t.e * p.b_estride;
  }
  la.init(A, A, p.lda, t.m_lo, t.m_hi, t.k_lo, t.k_hi, 0, tid, alt ? nullptr : p.a_rows);
  // columns are bounded in the B source's column space
  lb.init(B0, B1, p.ldb, t.n0, p.N, t.k_lo, t.k_hi, p.k_split, tid, nullptr);
}

// The MFMAs of one K slice: A tile at `as` ([BM] rows), B tile right after it.
// Wave (wm, wn) owns a (BM/WGM) x (BN/WGN) block of 32x32 accumulators; with
// the gate|up halves (B2_NHALF) its first FN/2 column blocks are gate columns
// and the last FN/2 the matching up columns.  The operand fragments of step
// ks+1 are read from LDS before the MFMAs of step ks are issued, so the LDS
// latency is hidden behind the matrix cores even with one wave per SIMD.
template <int BM, int BN, int WGM, int WGN, int AM, int BMD, int B2, bool SKIP, int FM, int FN>
__device__ __forceinline__ void load_frags(bf16x8 (&af)[FM], bf16x8 (&bfg)[FN], const bf16_t* as,
                                           int ks, int wm, int wn, int lane, int rows) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  const bf16_t* bs = as + BM * BK;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int base = wm * WTM + i * 32;
    if (SKIP && base >= rows) continue;  // a block of padding rows: no reads, no MFMAs
    if constexpr (AM == A_KC) af[i] = frag_kc(as, base, ks, lane);
    else af[i] = frag_kn<BM>(as, base, ks, lane);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int base;
    if constexpr (B2 == B2_NHALF)
      base = (j < FN / 2) ? (wn * (WTN / 2) + j * 32) : (BN / 2 + wn * (WTN / 2) + (j - FN / 2) * 32);
    else
      base = wn * WTN + j * 32;
    if constexpr (BMD == B_KC) bfg[j] = frag_kc(bs, base, ks, lane);
    else bfg[j] = frag_kn<BN>(bs, base, ks, lane);
  }
}

// `rows`: the tile's valid rows.  With PIPE, 32-row blocks at or past it are
// skipped (the other form computes padding rows too: testing for them there
// cost more registers than it saved).
struct NoHook {
  template <typename K>
  __device__ __forceinline__ void operator()(K) const {}
};

// `hook(integral_constant<ks>)` runs before MFMA step ks (the other form);
// with `active` false only the hooks run.
// RSKIP (PIPE only): test the row blocks against `rows` at all; GEMMs whose
// tiles are always full (the weight gradients: M is d or I) leave it off, so
// that the slice is straight-line code (the tests split it into small blocks
// the scheduler cannot interleave across).
template <int BM, int BN, int WGM, int WGN, int AM, int BMD, int B2, bool PIPE = false,
          bool RSKIP = true, int FM, int FN, typename Hook = NoHook>
__device__ __forceinline__ void mma_slice(f32x16 (&acc)[FM][FN], const bf16_t* as, int wm, int wn,
                                          int lane, int rows, Hook hook = Hook(),
                                          bool active = true) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static_assert(FM == WTM / 32 && FN == WTN / 32, "accumulator blocks match the wave tile");
  constexpr int KS = BK / 16;
  if constexpr (PIPE) {
    bf16x8 af[2][FM], bfg[2][FN];
    load_frags<BM, BN, WGM, WGN, AM, BMD, B2, RSKIP>(af[0], bfg[0], as, 0, wm, wn, lane, rows);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS)
        load_frags<BM, BN, WGM, WGN, AM, BMD, B2, RSKIP>(af[(ks + 1) & 1], bfg[(ks + 1) & 1], as,
                                                         ks + 1, wm, wn, lane, rows);
      // keep the next step's reads above this step's MFMAs (the scheduler
      // would otherwise move each read down to its first use)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (RSKIP && wm * WTM + i * 32 >= rows) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[ks & 1][j], af[ks & 1][i],
                                                             acc[i][j], 0, 0, 0);
      }
    }
  } else {
    auto kstep = [&](auto ksc) __attribute__((always_inline)) {
      constexpr int ks = decltype(ksc)::value;
      hook(ksc);
      if (!active) return;
      bf16x8 af[FM], bfg[FN];
      load_frags<BM, BN, WGM, WGN, AM, BMD, B2, false>(af, bfg, as, ks, wm, wn, lane, BM);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[j], af[i], acc[i][j], 0, 0, 0);
    };
    [&]<int... Ks>(std::integer_sequence<int, Ks...>) __attribute__((always_inline)) {
      (kstep(std::integral_constant<int, Ks>{}), ...);
    }(std::make_integer_sequence<int, KS>{});
  }
}

// Epilogue shared by the bf16 kernels.  Lane holds C[m][n..n+3] of every
// 32x32 block of its wave tile: m = row (lane & 31), n = 8q + 4 (lane >> 5).
template <int FM, int FN, int WTM, int WTN, int GMD, int EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x16 (&acc)[FM][FN], int m_lo,
                                         int m_hi, int n0, int e, int wm, int wn, int lane) {
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m_lo + wm * WTM + i * 32 + (lane & 31);
    if (m >= m_hi) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      bf16_t* H = static_cast<bf16_t*>(p.C0);
      bf16_t* Aout = static_cast<bf16_t*>(p.C2);
      const int64_t I = p.I;
#pragma unroll
      for (int jp = 0; jp < FN / 2; ++jp) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * (WTN / 2) + jp * 32 + 8 * q + 4 * half;
          if (n >= I) continue;
          float g[4], u[4], a[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            g[s] = acc[i][jp][4 * q + s];
            u[s] = acc[i][jp + FN / 2][4 * q + s];
            a[s] = g[s] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[s])) * u[s];
          }
          if (H) {
            *reinterpret_cast<uint2*>(H + m * 2 * I + n) = make_uint2(pack_bf2(g[0], g[1]), pack_bf2(g[2], g[3]));
            *reinterpret_cast<uint2*>(H + m * 2 * I + I + n) = make_uint2(pack_bf2(u[0], u[1]), pack_bf2(u[2], u[3]));
          }
          *reinterpret_cast<uint2*>(Aout + m * I + n) = make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int n = n0 + wn * WTN + j * 32 + 8 * q + 4 * half;
          if (n >= p.N) continue;
          float v[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = acc[i][j][4 * q + s];
          if constexpr (EPI == EPI_STORE) {
            bf16_t* C = static_cast<bf16_t*>(p.C0);
            if (p.n_split > 0 && n >= p.n_split) { C = static_cast<bf16_t*>(p.C1); n -= p.n_split; }
            if (GMD == G_KROWS) C += (int64_t)e * p.c_estride;
            *reinterpret_cast<uint2*>(C + (int64_t)m * p.ldc + n) =
                make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
          } else if constexpr (EPI == EPI_ACCUM) {
            bf16_t* C = static_cast<bf16_t*>(p.C0) + (int64_t)m * p.ldc + n;
            uint2 o = *reinterpret_cast<const uint2*>(C);
            float w0 = bf2f((bf16_t)(o.x & 0xffff)) + v[0], w1 = bf2f((bf16_t)(o.x >> 16)) + v[1];
            float w2 = bf2f((bf16_t)(o.y & 0xffff)) + v[2], w3 = bf2f((bf16_t)(o.y >> 16)) + v[3];
            *reinterpret_cast<uint2*>(C) = make_uint2(pack_bf2(w0, w1), pack_bf2(w2, w3));
          } else if constexpr (EPI == EPI_F32_BIAS) {
            float* C = static_cast<float*>(p.C0) + (int64_t)m * p.ldc + n;
            if (GMD == G_KROWS) C += (int64_t)e * p.c_estride;
            if (p.bias) {
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] += p.bias[n + s];
            }
            *reinterpret_cast<float4*>(C) = make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_DSWIGLU) {
            const bf16_t* H = static_cast<const bf16_t*>(p.aux);
            bf16_t* dH = static_cast<bf16_t*>(p.C0);
            const int64_t I = p.I;
            if (p.row_gate && !reads_alt(p)) {  // dA rows of g * dY[t]: the gate weight here
              const float gw = p.row_gate[p.row_slot[m]];
#pragma unroll
              for (int s = 0; s < 4; ++s) v[s] *= gw;
            }
            uint2 hg = *reinterpret_cast<const uint2*>(H + (int64_t)m * 2 * I + n);
            uint2 hu = *reinterpret_cast<const uint2*>(H + (int64_t)m * 2 * I + I + n);
            float g[4] = {bf2f((bf16_t)(hg.x & 0xffff)), bf2f((bf16_t)(hg.x >> 16)),
                          bf2f((bf16_t)(hg.y & 0xffff)), bf2f((bf16_t)(hg.y >> 16))};
            float u[4] = {bf2f((bf16_t)(hu.x & 0xffff)), bf2f((bf16_t)(hu.x >> 16)),
                          bf2f((bf16_t)(hu.y & 0xffff)), bf2f((bf16_t)(hu.y >> 16))};
            float dg[4], du[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[s]));
              dg[s] = v[s] * u[s] * sg * (1.0f + g[s] * (1.0f - sg));
              du[s] = v[s] * g[s] * sg;
            }
            *reinterpret_cast<uint2*>(dH + (int64_t)m * 2 * I + n) =
                make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(dH + (int64_t)m * 2 * I + I + n) =
                make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          }
        }
      }
    }
  }
}

// 16-byte result chunks of a block whose rows start at element offset `row0`
// of C0 / C1 and whose columns are [n_lo, n_hi): columns >= n_split go to C1
// at column - n_split.  A block on one side of n_split (the usual case) takes
// one buffer store per chunk; a block across it takes two masked ones.  A
// masked lane gets an out-of-range offset and its store is dropped.
struct BlockOut {
  __amdgpu_buffer_rsrc_t rs0, rs1;
  int shift;      // column shift of a one-sided block
  bool straddle;  // columns on both sides of n_split
  __device__ __forceinline__ BlockOut(const GemmParams& p, bf16_t* C0, bf16_t* C1, int64_t row0,
                                      int n_lo, int n_hi) {
    const bool split = p.n_split > 0;
    straddle = split && n_lo < p.n_split && n_hi > p.n_split;
    const bool upper = split && n_lo >= p.n_split;
    shift = upper ? p.n_split : 0;
    rs0 = make_rsrc((upper ? C1 : C0) + row0);
    rs1 = make_rsrc((C1 ? C1 : C0) + row0);
    if (straddle) rs0 = make_rsrc(C0 + row0);
  }
  template <int CPOL>
  __device__ __forceinline__ void store(const GemmParams& p, uint4 v, int r, int n, bool ok) const {
    const u32x4 d = __builtin_bit_cast(u32x4, v);
    if (!straddle) {
      const int off = (int)(((int64_t)r * p.ldc + n - shift) * 2);
      __builtin_amdgcn_raw_buffer_store_b128(d, rs0, ok ? off : OOB, 0, CPOL);
    } else {
      const bool hi = n >= p.n_split;
      const int off = (int)(((int64_t)r * p.ldc + n - (hi ? p.n_split : 0)) * 2);
      __builtin_amdgcn_raw_buffer_store_b128(d, rs0, ok && !hi ? off : OOB, 0, CPOL);
      __builtin_amdgcn_raw_buffer_store_b128(d, rs1, ok && hi ? off : OOB, 0, CPOL);
    }
  }
};

// Result staging in LDS: besides the chunk swizzle, the two 8-byte halves of
// a 16-byte chunk are swapped in rows where stage_swap(r), so that the 32
// lanes of an accumulator write (rows r..r+31, one 8-byte half each) hit 32
// different 8-byte bank groups instead of 16; whole-chunk readers and writers
// swap them back with swap_halves.
__device__ __forceinline__ int stage_swap(int r) { return ((r >> 3) ^ (r >> 4)) & 1; }
__device__ __forceinline__ uint4 swap_halves(uint4 v, int s) { return s ? make_uint4(v.z, v.w, v.x, v.y) : v; }

// Plain-store epilogue staged through LDS: the wave tiles are written to LDS
// as bf16, then every store instruction writes whole 16-byte chunks of
// consecutive columns (full cache lines per row) instead of 8-byte pieces
// scattered over 32 rows.  16-byte chunk c of LDS row r sits at c ^ (r & 15).
// `lds` holds BM * BN / ROUNDS bf16: the tile passes through it in ROUNDS
// bands of rows (WGM / ROUNDS wave rows each).  The caller synchronises before
// it reuses `lds`.
template <int BM, int BN, int WGM, int FM, int FN, int WTM, int WTN, int NT, int GMD, int ROUNDS>
__device__ __forceinline__ void epilogue_store_staged(const GemmParams& p, f32x16 (&acc)[FM][FN],
                                                      bf16_t* lds, int m_lo, int m_hi, int n0,
                                                      int e, int wm, int wn, int lane, int tid) {
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  static_assert(CPR >= 16, "swizzle needs 16 chunks per row");
  static_assert(WGM % ROUNDS == 0, "bands of whole wave rows");
  constexpr int WPR = WGM / ROUNDS;  // wave rows per band
  constexpr int RB = WPR * WTM;      // tile rows per band
  const int half = lane >> 5;
  bf16_t* C0 = static_cast<bf16_t*>(p.C0);
  bf16_t* C1 = static_cast<bf16_t*>(p.C1);
  if (GMD == G_KROWS) {
    C0 += (int64_t)e * p.c_estride;
    if (C1) C1 += (int64_t)e * p.c_estride;
  }
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    if (rd > 0) __syncthreads();  // the previous band has been read back
    if (wm / WPR == rd) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = (wm - rd * WPR) * WTM + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = wn * WTN + j * 32 + 8 * q + 4 * half;
            const int c = (n >> 3) ^ (r & 15);
            *reinterpret_cast<uint2*>(lds + r * BN + c * 8 + ((n & 7) ^ (stage_swap(r) << 2))) =
                make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                           pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
          }
        }
      }
    }
    __syncthreads();
    // all LDS reads first (every lane's address is inside the band), then
    // the masked stores
    constexpr int NQ = (RB * CPR + NT - 1) / NT;
    uint4 v[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = min(i * NT + tid, RB * CPR - 1);
      const int r = q / CPR, c = q % CPR;
      v[i] = swap_halves(*reinterpret_cast<const uint4*>(lds + r * BN + (c ^ (r & 15)) * 8), stage_swap(r));
    }
    // buffer stores relative to the band's first row: a masked lane gets an
    // out-of-range offset and its store is dropped, so no lane branches
    const BlockOut bo(p, C0, C1, (int64_t)(m_lo + rd * RB) * p.ldc, n0, n0 + BN);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = i * NT + tid;
      const int r = q / CPR, c = q % CPR;
      const int n = n0 + c * 8;
      const bool ok = (RB * CPR % NT == 0 || q < RB * CPR) && m_lo + rd * RB + r < m_hi && n < p.N;
      bo.store<0>(p, v[i], r, n, ok);
    }
  }
}

// Staged activation epilogues.  The tile passes through LDS in bands of one
// wave row (WTM rows); each band array is [WTM][W] bf16 (W = 128 or 256) with 16-byte chunk
// c of row r at c ^ (r & 15), so that memory is read and written in whole
// 16-byte chunks of consecutive columns (full cache lines per row) instead
// of 8-byte pieces spread over 32 rows.
// (halves swapped by stage_swap as in the plain staging).  band_off gives
// element n of row r; band_chunk the start of whole chunk c.
template <int W = 128>
__device__ __forceinline__ int band_off(int r, int n) {
  return r * W + (((n >> 3) ^ (r & 15)) << 3) + ((n & 7) ^ (stage_swap(r) << 2));
}
template <int W = 128>
__device__ __forceinline__ int band_chunk(int r, int c) { return r * W + ((c ^ (r & 15)) << 3); }

// SwiGLU: gate columns n0 .. n0+127 and the matching up columns of the tile
// give H = [Hg | Hu] (optional) and A = silu(Hg) * Hu.
template <int BM, int BN, int WGM, int FM, int FN, int WTM, int WTN, int NT>
__device__ __forceinline__ void epilogue_swiglu_staged(const GemmParams& p, f32x16 (&acc)[FM][FN],
                                                       bf16_t* lds, int m_lo, int m_hi, int n0,
                                                       int wm, int wn, int lane, int tid) {
  constexpr int HC = BN / 2;  // columns per half (128)
  constexpr int BAND = WTM * HC;
  bf16_t* Gs = lds;
  bf16_t* Us = lds + BAND;
  bf16_t* As = lds + 2 * BAND;
  bf16_t* H = static_cast<bf16_t*>(p.C0);
  bf16_t* Aout = static_cast<bf16_t*>(p.C2);
  const int64_t I = p.I;
  const int half = lane >> 5;
#pragma unroll
  for (int rd = 0; rd < WGM; ++rd) {
    if (rd > 0) __syncthreads();  // the previous band has been read back
    if (wm == rd) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = i * 32 + (lane & 31);
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = wn * (WTN / 2) + jp * 32 + 8 * q + 4 * half;
            float g[4], u[4], a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              g[t] = acc[i][jp][4 * q + t];
              u[t] = acc[i][jp + FN / 2][4 * q + t];
              a[t] = g[t] * __builtin_amdgcn_rcpf(1.0f + __expf(-g[t])) * u[t];
            }
            const int o = band_off(r, n);
            *reinterpret_cast<uint2*>(Gs + o) = make_uint2(pack_bf2(g[0], g[1]), pack_bf2(g[2], g[3]));
            *reinterpret_cast<uint2*>(Us + o) = make_uint2(pack_bf2(u[0], u[1]), pack_bf2(u[2], u[3]));
            *reinterpret_cast<uint2*>(As + o) = make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
          }
      }
    }
    __syncthreads();
    const int mb = m_lo + rd * WTM;
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(Aout + (int64_t)mb * I + n0);
    const __amdgpu_buffer_rsrc_t rsg = make_rsrc((H ? H : Aout) + (int64_t)mb * 2 * I + n0);
    const __amdgpu_buffer_rsrc_t rsu = make_rsrc((H ? H : Aout) + (int64_t)mb * 2 * I + I + n0);
#pragma unroll
    for (int q0 = 0; q0 < WTM * (HC / 8); q0 += NT) {
      const int q = q0 + tid;
      const int r = q / (HC / 8), c = q % (HC / 8);
      const bool ok = mb + r < m_hi && n0 + c * 8 < I;
      const int o = band_chunk(r, c), sw = stage_swap(r);
      const u32x4 va = __builtin_bit_cast(u32x4, swap_halves(*reinterpret_cast<const uint4*>(As + o), sw));
      __builtin_amdgcn_raw_buffer_store_b128(va, rsa, ok ? (int)(((int64_t)r * I + c * 8) * 2) : OOB, 0, 0);
      if (H) {
        const u32x4 vg = __builtin_bit_cast(u32x4, swap_halves(*reinterpret_cast<const uint4*>(Gs + o), sw));
        const u32x4 vu = __builtin_bit_cast(u32x4, swap_halves(*reinterpret_cast<const uint4*>(Us + o), sw));
        const int oh = ok ? (int)(((int64_t)r * 2 * I + c * 8) * 2) : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(vg, rsg, oh, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(vu, rsu, oh, 0, 0);
      }
    }
  }
}

// dSwiGLU: acc = dA for columns n0 .. n0+BN-1; reads H = [Hg | Hu] of those
// columns and writes dH = [dHg | dHu].
template <int BM, int BN, int WGM, int FM, int FN, int WTM, int WTN, int NT>
__device__ __forceinline__ void epilogue_dswiglu_staged(const GemmParams& p, f32x16 (&acc)[FM][FN],
                                                        bf16_t* lds, int m_lo, int m_hi, int n0,
                                                        int wm, int wn, int lane, int tid) {
  constexpr int BAND = WTM * BN;
  constexpr int CPR = BN / 8;
  bf16_t* Gs = lds;
  bf16_t* Us = lds + BAND;
  const bf16_t* H = static_cast<const bf16_t*>(p.aux);
  bf16_t* dH = static_cast<bf16_t*>(p.C0);
  const int64_t I = p.I;
  const int half = lane >> 5;
#pragma unroll
  for (int rd = 0; rd < WGM; ++rd) {
    const int mb = m_lo + rd * WTM;
    const int64_t hrow = (int64_t)mb * 2 * I + n0;
    // 1. the band's Hg and Hu into LDS (rows past m_hi and columns past I read zeros)
    {
      const __amdgpu_buffer_rsrc_t rsg = make_rsrc(H + hrow);
      const __amdgpu_buffer_rsrc_t rsu = make_rsrc(H + hrow + I);
      constexpr int NQ = (WTM * CPR + NT - 1) / NT;
      uint4 vg[NQ], vu[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int q = i * NT + tid;
        const int r = q / CPR, c = q % CPR;
        const bool ok = (WTM * CPR % NT == 0 || q < WTM * CPR) && mb + r < m_hi && n0 + c * 8 < I;
        const int off = ok ? (int)(((int64_t)r * 2 * I + c * 8) * 2) : OOB;
        vg[i] = buf_load16<0>(rsg, off, 0);
        vu[i] = buf_load16<0>(rsu, off, 0);
      }
      if (rd > 0) __syncthreads();  // the previous band has been read back
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int q = i * NT + tid;
        if (WTM * CPR % NT == 0 || q < WTM * CPR) {
          const int r = q / CPR, c = q % CPR;
          *reinterpret_cast<uint4*>(Gs + band_chunk<BN>(r, c)) = swap_halves(vg[i], stage_swap(r));
          *reinterpret_cast<uint4*>(Us + band_chunk<BN>(r, c)) = swap_halves(vu[i], stage_swap(r));
        }
      }
    }
    __syncthreads();
    // 2. the band's waves turn (dA, Hg, Hu) into (dHg, dHu) in place (dA rows
    // of g * dY[t] take their gate weight g here; rows past m_hi read the
    // last valid row's and are not stored).  With dg_part, each 32-column
    // block's share of the gate gradient, sum of dA0 * silu(Hg) Hu over the
    // block (dA0: before the gate weight), goes out too: a lane sums its 16
    // columns, the lane 32 apart (same row, the other 16) adds its sum.
    const bool dgw = p.dg_part != nullptr && !reads_alt(p);
    if (wm == rd) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = i * 32 + (lane & 31);
        const float gw = p.row_gate && !reads_alt(p) ? p.row_gate[p.row_slot[min(mb + r, m_hi - 1)]]
                                                     : 1.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          float dgs = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = wn * WTN + j * 32 + 8 * q + 4 * half;
            const int o = band_off<BN>(r, n);
            const uint2 hg = *reinterpret_cast<const uint2*>(Gs + o);
            const uint2 hu = *reinterpret_cast<const uint2*>(Us + o);
            const float g[4] = {bf2f((bf16_t)(hg.x & 0xffff)), bf2f((bf16_t)(hg.x >> 16)),
                                bf2f((bf16_t)(hg.y & 0xffff)), bf2f((bf16_t)(hg.y >> 16))};
            const float u[4] = {bf2f((bf16_t)(hu.x & 0xffff)), bf2f((bf16_t)(hu.x >> 16)),
                                bf2f((bf16_t)(hu.y & 0xffff)), bf2f((bf16_t)(hu.y >> 16))};
            float dg[4], du[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float a0 = acc[i][j][4 * q + t];
              const float v = a0 * gw;
              const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[t]));
              dg[t] = v * u[t] * sg * (1.0f + g[t] * (1.0f - sg));
              du[t] = v * g[t] * sg;
              dgs = fmaf(a0, g[t] * sg * u[t], dgs);
            }
            *reinterpret_cast<uint2*>(Gs + o) = make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(Us + o) = make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          }
          if (dgw) {
            dgs += __shfl_xor(dgs, 32, 64);
            const int blk = (n0 + wn * WTN + j * 32) / 32;
            if (half == 0 && mb + r < m_hi && blk < p.dg_stride)
              p.dg_part[(int64_t)(mb + r) * p.dg_stride + blk] = dgs;
          }
        }
      }
    }
    __syncthreads();
    // 3. whole chunks out
    const __amdgpu_buffer_rsrc_t rsg = make_rsrc(dH + hrow);
    const __amdgpu_buffer_rsrc_t rsu = make_rsrc(dH + hrow + I);
#pragma unroll
    for (int q0 = 0; q0 < WTM * CPR; q0 += NT) {
      const int q = q0 + tid;
      const int r = q / CPR, c = q % CPR;
      const bool ok = (WTM * CPR % NT == 0 || q < WTM * CPR) && mb + r < m_hi && n0 + c * 8 < I;
      const int off = ok ? (int)(((int64_t)r * 2 * I + c * 8) * 2) : OOB;
      const int o = band_chunk<BN>(r, c), sw = stage_swap(r);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, swap_halves(*reinterpret_cast<const uint4*>(Gs + o), sw)), rsg, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, swap_halves(*reinterpret_cast<const uint4*>(Us + o), sw)), rsu, off, 0, 0);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM.  WGM x WGN waves, each owning a (BM/WGM) x
// (BN/WGN) block of 32x32 MFMA tiles.  P register stages: while the
// MFMAs work on K slice kt from LDS, slice kt+1 is written to the other LDS
// buffer and the loads of slices kt+2 .. kt+P are in flight.
// With the gate|up halves (B2_NHALF) the first FN/2 column blocks of a wave
// are gate columns and the last FN/2 the matching up columns.
// ---------------------------------------------------------------------------
// Refill loads of gemm_bf16_kernel's steady state: 0 = all at the top of the
// step; 1 = two parts, before MFMA steps 0 and 2; 2 = four parts, one per MFMA
// step (build-time tunable).  Eight waves sending a whole slice of loads at
// once fill the memory pipeline's address queue and stall their own MFMA
// issue; parts spread the loads over the step.
#ifndef MOE_LOAD_SPLIT
#define MOE_LOAD_SPLIT 2
#endif
template <int BM, int BN, int WGM, int WGN, int P, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile of at least 32x32");
  static_assert(B2 != B2_NHALF || FN % 2 == 0, "gate|up halves need an even block count");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- which tile
  const int count = tile_count<GMD>(p);
  if ((int)blockIdx.x >= count) return;
  const TileDesc t = tile_desc<BM, BN, GMD, B2>(p, remap_xcd(blockIdx.x, count));
  const int e = t.e, m_lo = t.m_lo, m_hi = t.m_hi, n0 = t.n0, k_lo = t.k_lo, k_hi = t.k_hi;
  // A wave whose rows all lie at or past the tile's last valid row (the
  // ragged last tile of a group) skips the MFMAs; it still loads and stores
  // its share of each slice and takes part in every barrier.
  const bool wave_rows = wm * WTM < m_hi - m_lo;

  typedef typename Loaders<BM, BN, NT, AM, BMD, GMD, B2, gathers_a(ROLE), full_k(ROLE)>::LA LA;
  typedef typename Loaders<BM, BN, NT, AM, BMD, GMD, B2, gathers_a(ROLE), full_k(ROLE)>::LB LB;
  LA la;
  LB lb;
  typename LA::Data da[P];
  typename LB::Data db[P];
  init_loaders<GMD, B2>(p, t, la, lb, tid);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (k_hi - k_lo + BK - 1) / BK;
  // The first P slices load (and slice 0 is stored) unconditionally: slices
  // past the K range read as zeros without touching memory.  Guarding them
  // would leave loads that are never waited for on the guarded path, and the
  // compiler, merging that path into the loop, would then wait for the
  // previous step's loads at the top of every step.
#pragma unroll
  for (int s = 0; s < P; ++s) {
    la.load(da[s], s * BK, tid);
    lb.load(db[s], s * BK, tid);
  }
  LA::store(da[0], smem, tid);
  LB::store(db[0], smem + BM * BK, tid);
  __syncthreads();

  // One K slice: refill the register slot of slice kt with slice kt+P, multiply
  // slice kt from LDS, write slice kt+1 (loaded P-1 slices ago) to the other
  // LDS buffer, barrier.  U = kt mod P is a compile-time constant.
  auto step = [&](auto Uc, auto Sc, int kt, bool do_load, bool do_store)
                  __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    if constexpr (!decltype(Sc)::value) {
      if (do_load) {
        la.load(da[U], (kt + P) * BK, tid);
        lb.load(db[U], (kt + P) * BK, tid);
      }
      // keep the refill loads at the top of the step: the scheduler would
      // otherwise sink them below the MFMAs and expose their latency
      __builtin_amdgcn_sched_barrier(0);
      if (wave_rows)
        mma_slice<BM, BN, WGM, WGN, AM, BMD, B2>(acc, smem + (kt & 1) * (BM + BN) * BK, wm, wn,
                                                 lane, m_hi - m_lo);
    } else {
      // steady state (every step loads): the refill loads go out in parts
      // between the MFMA steps, each part pinned in place
      auto hook = [&](auto ksc) __attribute__((always_inline)) {
        constexpr int ks = decltype(ksc)::value;
        constexpr int NJ = MOE_LOAD_SPLIT == 1 ? 2 : 4;
        if constexpr (ks % (4 / NJ) == 0) {
          __builtin_amdgcn_sched_barrier(0);
          la.template load_part<ks / (4 / NJ), NJ>(da[U], (kt + P) * BK, tid);
          lb.template load_part<ks / (4 / NJ), NJ>(db[U], (kt + P) * BK, tid);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      __builtin_amdgcn_sched_barrier(0);
      mma_slice<BM, BN, WGM, WGN, AM, BMD, B2>(acc, smem + (kt & 1) * (BM + BN) * BK, wm, wn, lane,
                                               m_hi - m_lo, hook, wave_rows);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_store) {
      bf16_t* nxt = smem + ((kt + 1) & 1) * (BM + BN) * BK;
      LA::store(da[(U + 1) % P], nxt, tid);
      LB::store(db[(U + 1) % P], nxt + BM * BK, tid);
    }
    __syncthreads();
  };

  int kt0 = 0;
  // steady state: every step loads and stores
  for (; kt0 + 2 * P <= nk; kt0 += P) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
      (step(std::integral_constant<int, Us>{}, std::bool_constant<MOE_LOAD_SPLIT != 0>{}, kt0 + Us,
            true, true),
       ...);
    }(std::make_integer_sequence<int, P>{});
  }
  // drain: at most 2P-1 slices left
  [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
    ((kt0 + Us < nk ? step(std::integral_constant<int, Us % P>{}, std::false_type{}, kt0 + Us,
                           kt0 + Us + P < nk, kt0 + Us + 1 < nk)
                    : void()),
     ...);
  }(std::make_integer_sequence<int, 2 * P - 1>{});

#ifndef MOE_STAGED_STORE
#define MOE_STAGED_STORE 1
#endif
  // the two LDS buffers are free here (the last step ended with a barrier)
  constexpr int LDS_ELEMS = (BM + BN) * BK * 2;
  if constexpr (EPI == EPI_STORE && MOE_STAGED_STORE && BN / 8 >= 16 && BM * BN <= LDS_ELEMS)
    epilogue_store_staged<BM, BN, WGM, FM, FN, WTM, WTN, NT, GMD, 1>(p, acc, smem, m_lo, m_hi, n0, e,
                                                                    wm, wn, lane, tid);
  else if constexpr (EPI == EPI_SWIGLU && MOE_STAGED_STORE && BN / 16 == 16 &&
                     3 * WTM * (BN / 2) <= LDS_ELEMS)
    epilogue_swiglu_staged<BM, BN, WGM, FM, FN, WTM, WTN, NT>(p, acc, smem, m_lo, m_hi, n0, wm, wn,
                                                            lane, tid);
  else if constexpr (EPI == EPI_DSWIGLU && MOE_STAGED_STORE && (BN == 128 || BN == 256) &&
                     2 * WTM * BN <= LDS_ELEMS)
    epilogue_dswiglu_staged<BM, BN, WGM, FM, FN, WTM, WTN, NT>(p, acc, smem, m_lo, m_hi, n0, wm, wn,
                                                             lane, tid);
  else {
    // (the gate gradient's shares are written by the staged dSwiGLU epilogue only)
    static_assert(ROLE != R_DOWN_DGRAD_GATHER, "R_DOWN_DGRAD_GATHER needs the staged epilogue");
    epilogue<FM, FN, WTM, WTN, GMD, EPI>(p, acc, m_lo, m_hi, n0, e, wm, wn, lane);
  }
}

// ---------------------------------------------------------------------------
// Persistent bf16 MFMA grouped GEMM.  About as many workgroups as fit on the
// chip at once each run a fixed list of tiles back to back, and the K-slice
// pipeline of gemm_bf16_kernel (two register stages, two LDS buffers) runs on
// across tile boundaries: the first slices of the next tile are in flight
// while the current tile finishes its MFMAs and writes its result, so neither
// the pipeline fill nor the epilogue leaves the matrix cores idle.  This
// matters where a tile has few K slices (the weight gradients: K is the rows
// of one expert).
// Workgroup w runs on XCD w % 8 (the hardware's round-robin dispatch) and
// takes every (gridDim.x / 8)-th tile of the contiguous range of tile ids that
// its XCD owns, so tiles that share operands stay in one L2.  gridDim.x is a
// multiple of 8.  Tiles with no K slices (an expert with no rows in the weight
// gradients) are written as zeros.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_persistent_kernel(GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int BUF = (BM + BN) * BK;  // one LDS buffer (A slice, then B slice)
  static_assert(FM >= 1 && FN >= 1, "wave tile of at least 32x32");
  static_assert(B2 != B2_NHALF || FN % 2 == 0, "gate|up halves need an even block count");
  // plain stores are staged through the LDS buffer that the finished slice
  // frees, in bands of rows that fit into it
  constexpr bool STAGED = EPI == EPI_STORE && BN / 8 >= 16;
  constexpr int ROUNDS = (BM * BN + BUF - 1) / BUF;
  static_assert(!STAGED || (WGM % ROUNDS == 0 && BM * BN / ROUNDS <= BUF), "staging bands");
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- this workgroup's tiles: x_lo + pos for pos = slot, slot + S, ... < x_n
  const int count = tile_count<GMD>(p);
  const int xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD, S = gridDim.x / NXCD;
  int x_lo, x_n;
  xcd_tile_range<GMD>(p, count, xcd, x_lo, x_n);
  if (slot >= x_n) return;

  typedef typename Loaders<BM, BN, NT, AM, BMD, GMD, B2, gathers_a(ROLE), full_k(ROLE)>::LA LA;
  typedef typename Loaders<BM, BN, NT, AM, BMD, GMD, B2, gathers_a(ROLE), full_k(ROLE)>::LB LB;
  LA la;
  LB lb;
  typename LA::Data da[2];
  typename LB::Data db[2];

  f32x16 acc[FM][FN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  auto slices = [](const TileDesc& t) { return (t.k_hi - t.k_lo + BK - 1) / BK; };

  // Load cursor: the tile (position l_pos) and slice (l_ks of l_nk) whose
  // loads go out next.  Moves to the next tile with K slices and points the
  // loaders at it.
  int l_pos = slot, l_ks = 0, l_nk = 0;
  // Past the end, the cursor stays on the last slice index of the last tile
  // with slices (l_ks == l_nk), where the loads read nothing.
  auto load_seek = [&]() __attribute__((always_inline)) {
    for (; l_pos < x_n; l_pos += S) {
      const TileDesc t = tile_desc<BM, BN, GMD, B2>(p, x_lo + l_pos);
      const int nk = slices(t);
      if (nk > 0) {
        l_nk = nk;
        l_ks = 0;
        init_loaders<GMD, B2>(p, t, la, lb, tid);
        break;
      }
    }
  };
  int issued = 0;  // slices whose loads have gone out
  // Loads of the slice at the load cursor into register stage U.  Inside the
  // loop the loads go out unconditionally: past the last slice the loaders
  // still point at the last tile, and a slice beyond its K range reads zeros
  // through the range check without touching memory.  (A load under a branch
  // would make the compiler wait for every load in flight at the join.)
  auto issue = [&](auto Uc, bool first) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    if (!first || l_pos < x_n) {
      la.load(da[U], l_ks * BK, tid);
      lb.load(db[U], l_ks * BK, tid);
    }
    if (l_pos < x_n) {
      ++issued;
      if (++l_ks == l_nk) {
        l_pos += S;
        load_seek();
      }
    }
  };

  // Compute cursor: the tile being accumulated (ct, position c_pos) and its
  // slice count.
  int c_pos = slot, c_ks = 0, c_nk = 0;
  TileDesc ct;
  auto finish = [&](bf16_t* stage) __attribute__((always_inline)) {
    if constexpr (STAGED) {
      epilogue_store_staged<BM, BN, WGM, FM, FN, WTM, WTN, NT, GMD, ROUNDS>(
          p, acc, stage, ct.m_lo, ct.m_hi, ct.n0, ct.e, wm, wn, lane, tid);
      __syncthreads();  // `stage` is read back before anyone refills it
    } else {
      epilogue<FM, FN, WTM, WTN, GMD, EPI>(p, acc, ct.m_lo, ct.m_hi, ct.n0, ct.e, wm, wn, lane);
    }
  };
  // Move to the next tile with K slices; tiles without any are written as
  // zeros on the way (acc is zero here).
  auto compute_seek = [&](bf16_t* stage) __attribute__((always_inline)) {
    for (; c_pos < x_n; c_pos += S) {
      ct = tile_desc<BM, BN, GMD, B2>(p, x_lo + c_pos);
      c_nk = slices(ct);
      c_ks = 0;
      if (c_nk > 0) break;
      finish(stage);
    }
  };

  zero_acc();
  load_seek();
  issue(std::integral_constant<int, 0>{}, true);
  issue(std::integral_constant<int, 1>{}, true);
  compute_seek(smem);
  if (issued == 0) return;  // every tile of this workgroup was empty
  LA::store(da[0], smem, tid);
  LB::store(db[0], smem + BM * BK, tid);
  __syncthreads();

  // One K slice g (U = g mod 2 is both its register stage and its LDS
  // buffer): send the loads of slice g+2 into stage U, multiply slice g from
  // buffer U, write slice g+1 (stage 1-U) into buffer 1-U, barrier.  After the
  // last slice of a tile, write the tile out, staging through buffer U.
  // Returns false once every tile is done.
  int g = 0;
  auto step = [&](auto Uc) __attribute__((always_inline)) -> bool {
    constexpr int U = decltype(Uc)::value;
    issue(Uc, false);
    // keep the loads at the top of the step (the scheduler would sink them)
    __builtin_amdgcn_sched_barrier(0);
    mma_slice<BM, BN, WGM, WGN, AM, BMD, B2>(acc, smem + U * BUF, wm, wn, lane, ct.m_hi - ct.m_lo);
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < issued) {
      LA::store(da[1 - U], smem + (1 - U) * BUF, tid);
      LB::store(db[1 - U], smem + (1 - U) * BUF + BM * BK, tid);
    }
    __syncthreads();
    ++g;
    if (++c_ks < c_nk) return true;
    finish(smem + U * BUF);
    zero_acc();
    c_pos += S;
    compute_seek(smem + U * BUF);
    return c_pos < x_n;
  };
  while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
  }
}

// ---------------------------------------------------------------------------
// Combine fused into the down projection's epilogue (R_DOWN_FWD_COMBINE).
// A compute wave has just stored its block of Yp: rows [mb, m_hi) (one per
// lane), the 64 columns from nb.  Those stores used the device-coherent cache
// policy (sc1: written through to the point every XCD reads from).  Per row,
// the wave waits for its stores, then bumps the integer arrival counter of
// (the row's token, the column block); the wave whose increment completes a
// token's count (its kept slots) is the last writer of that token's row
// blocks, and computes y[t] for those 64 columns: sum over the token's slots
// in ascending j of w[t,j] * Yp[inv[t,j]] (device-coherent loads), in fp32,
// the same operations in the same order as the combine kernel, so y is
// bit-identical to moe_combine's.  Deterministic: counters are integers and
// the sum order does not depend on who arrives last.
// ---------------------------------------------------------------------------
constexpr int CMB_STORE_CPOL = 16;  // sc1: device-coherent store
constexpr int CMB_LOAD_CPOL = 16;   // sc1: device-coherent load

__device__ __forceinline__ void combine_rows(const GemmParams& p, int mb, int m_hi, int nb,
                                             int lane) {
  if (nb >= p.N) return;  // a block of padding columns (uniform)
  const int ncb = p.N >> 6;
  const int cb = nb >> 6;
  // this wave's stores of its block are complete before its counters move
  // (vmcnt(0); the exp and lgkm counters left as they are)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  const int row = mb + lane;
  int tok = 0;
  bool last = false;
  if (row < m_hi) {
    tok = p.cmb_tok[row];
    const int old = __hip_atomic_fetch_add(p.cmb_cnt + (int64_t)tok * ncb + cb, 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == p.cmb_kept[tok] - 1;
  }
  // the reads below stay after the counter updates
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  uint64_t mask = __ballot(last);
  const __amdgpu_buffer_rsrc_t ryp = make_rsrc(static_cast<const bf16_t*>(p.C0) + nb);
  bf16_t* Y = static_cast<bf16_t*>(p.cmb_y);
  const int grp = lane >> 3, c = lane & 7;  // 8 tokens at a time, 8 chunks of 8 columns each
  const int k = p.cmb_k;
  while (mask) {  // uniform
    int r[8], n = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      r[g] = mask ? (int)__builtin_ctzll(mask) : 0;
      if (mask) { mask &= mask - 1; ++n; }
    }
    int my = r[0];
#pragma unroll
    for (int g = 1; g < 8; ++g) my = grp == g ? r[g] : my;
    const int t = __shfl(tok, my, 64);
    if (grp < n) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      for (int j0 = 0; j0 < k; j0 += 8) {
        int pj[8];
        float gj[8];
        uint4 v[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = j0 + jj;
          pj[jj] = j < k ? p.cmb_inv[(int64_t)t * k + j] : -1;
          gj[jj] = j < k ? p.cmb_w[(int64_t)t * k + j] : 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          v[jj] = buf_load16<CMB_LOAD_CPOL>(
              ryp, pj[jj] >= 0 ? (int)(((int64_t)pj[jj] * p.ldc + c * 8) * 2) : OOB, 0);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          if (pj[jj] < 0) continue;
          const uint32_t w4[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(gj[jj], __uint_as_float(w4[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(gj[jj], __uint_as_float(w4[i] & 0xffff0000u), acc[2 * i + 1]);
          }
        }
      }
      *reinterpret_cast<uint4*>(Y + (int64_t)t * p.N + nb + c * 8) =
          make_uint4(pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]), pack_bf2(acc[4], acc[5]),
                     pack_bf2(acc[6], acc[7]));
    }
  }
}

// ---------------------------------------------------------------------------
// Warp-specialised persistent bf16 MFMA GEMM.  Compute waves (WGM x WGN)
// only read LDS, run the MFMAs and write results; producer waves (NPW) only
// load K slices from memory into LDS, with PD slices in flight in their own
// registers.  On this hardware a wave's loads and stores retire in one
// in-order queue, so a wave that stores its result and then waits for its
// next slice also waits for the stores: here the compute waves write their
// finished blocks while the producer waves, which never store, keep the next
// slices coming.  Plain stores are staged through a private LDS area per
// compute wave (whole 16-byte chunks of consecutive columns); the other
// epilogues write from registers.  Tile order and the K-slice pipeline across
// tiles are those of gemm_bf16_persistent_kernel.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int NPW, int PD, int AM, int BMD, int GMD, int B2, int EPI,
          int ROLE>
__global__ __launch_bounds__(64 * (WGM * WGN + NPW)) void gemm_bf16_ws_kernel(GemmParams p) {
  static_assert(EPI != EPI_STORE || B2 != B2_NHALF, "plain stores need contiguous wave columns");
  constexpr int NC = WGM * WGN;       // compute waves
  constexpr int NTP = 64 * NPW;       // producer threads
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int BUF = (BM + BN) * BK;
  constexpr int SCPR = WTN / 8;       // 16-byte chunks per staged row
  static_assert(EPI != EPI_STORE || SCPR == 8 || SCPR == 16, "staged rows of 64 or 128 columns");
  constexpr int WST = EPI == EPI_STORE ? WTM * WTN : 0;  // staging elements per compute wave
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * BUF + NC * WST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= NC;
  const int wm = wave / WGN, wn = wave % WGN;  // compute waves only
  const int ptid = tid - NC * 64;              // producer waves only

  const int count = tile_count<GMD>(p);
  const int xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD, S = gridDim.x / NXCD;
  int x_lo, x_n;
  xcd_tile_range<GMD>(p, count, xcd, x_lo, x_n);
  if (slot >= x_n) return;
  auto slices = [](const TileDesc& t) { return (t.k_hi - t.k_lo + BK - 1) / BK; };

  // ---- producer state: loaders, PD register stages, load cursor
  static_assert(PD >= 2, "at least two register stages");
  typedef typename Loaders<BM, BN, NTP, AM, BMD, GMD, B2, gathers_a(ROLE), full_k(ROLE)>::LA LA;
  typedef typename Loaders<BM, BN, NTP, AM, BMD, GMD, B2, gathers_a(ROLE), full_k(ROLE)>::LB LB;
  LA la;
  LB lb;
  typename LA::Data da[PD];
  typename LB::Data db[PD];
  int l_pos = slot, l_ks = 0, l_nk = 0, issued = 0;
  auto load_seek = [&]() __attribute__((always_inline)) {
    for (; l_pos < x_n; l_pos += S) {
      const TileDesc t = tile_desc<BM, BN, GMD, B2>(p, x_lo + l_pos);
      const int nk = slices(t);
      if (nk > 0) {
        l_nk = nk;
        l_ks = 0;
        init_loaders<GMD, B2>(p, t, la, lb, ptid);
        break;
      }
    }
  };
  // see gemm_bf16_persistent_kernel: loads in the loop go out unconditionally
  auto issue = [&](auto Uc, bool first) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    if (!first || l_pos < x_n) {
      la.load(da[U], l_ks * BK, ptid);
      lb.load(db[U], l_ks * BK, ptid);
    }
    if (l_pos < x_n) {
      ++issued;
      if (++l_ks == l_nk) {
        l_pos += S;
        load_seek();
      }
    }
  };

  // ---- compute state: accumulators and the wave's block of the tile
  f32x16 acc[FM][FN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  bf16_t* stage = smem + 2 * BUF + (producer ? 0 : wave) * WST;
  // Write the wave's WTM x WTN block: accumulators -> private LDS area
  // (16-byte chunk c of row r at c ^ (r mod SCPR)) -> whole chunks to memory
  // with buffer stores (masked lanes get an out-of-range offset).
#ifndef MOE_WS_STAGED
#define MOE_WS_STAGED 1
#endif
  auto store_block = [&](const TileDesc& t) __attribute__((always_inline)) {
    if constexpr (EPI != EPI_STORE || !MOE_WS_STAGED) {
      epilogue<FM, FN, WTM, WTN, GMD, EPI>(p, acc, t.m_lo, t.m_hi, t.n0, t.e, wm, wn, lane);
      return;
    }
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = j * 32 + 8 * q + 4 * half;
          const int c = (n >> 3) ^ (r & (SCPR - 1));
          *reinterpret_cast<uint2*>(stage + r * WTN + c * 8 + (n & 7)) =
              make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                         pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
    }
    // the wave's own LDS writes and reads execute in order; keep the compiler
    // from moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    constexpr int NQ = WTM * SCPR / 64;  // chunks per lane
    constexpr int QB = NQ < 8 ? NQ : 8;   // chunks per batch (bounds the registers)
    bf16_t* C0 = static_cast<bf16_t*>(p.C0);
    bf16_t* C1 = static_cast<bf16_t*>(p.C1);
    if (GMD == G_KROWS) {
      C0 += (int64_t)t.e * p.c_estride;
      if (C1) C1 += (int64_t)t.e * p.c_estride;
    }
    const int mb = t.m_lo + wm * WTM;
    const int nb = t.n0 + wn * WTN;
    const BlockOut bo(p, C0, C1, (int64_t)mb * p.ldc, nb, nb + WTN);
#pragma unroll
    for (int i0 = 0; i0 < NQ; i0 += QB) {
      uint4 v[QB];
#pragma unroll
      for (int i = 0; i < QB; ++i) {
        const int q = (i0 + i) * 64 + lane;
        const int r = q / SCPR, c = q % SCPR;
        v[i] = *reinterpret_cast<const uint4*>(stage + r * WTN + (c ^ (r & (SCPR - 1))) * 8);
      }
#pragma unroll
      for (int i = 0; i < QB; ++i) {
        const int q = (i0 + i) * 64 + lane;
        const int r = q / SCPR, c = q % SCPR;
        const int n = nb + c * 8;
        // weight gradients are not read again soon: stream them past the
        // caches; other results (read by the next kernel) stay cacheable;
        // with the fused combine, device-coherent (other XCDs read them)
        bo.store<GMD == G_KROWS ? MOE_OUT_CPOL : ROLE == R_DOWN_FWD_COMBINE ? CMB_STORE_CPOL : 0>(
            p, v[i], r, n, mb + r < t.m_hi && n < p.N);
      }
    }
    if constexpr (ROLE == R_DOWN_FWD_COMBINE) {
      static_assert(WTM == 64 && WTN == 64, "one row per lane, 64-column counter blocks");
      combine_rows(p, mb, t.m_hi, nb, lane);
    }
  };

  // ---- compute cursor (every wave keeps it; it decides when the loop ends)
  int c_pos = slot, c_ks = 0, c_nk = 0;
  TileDesc ct;
  // (the producer and compute forms are separate instances, so that the
  // producer loop never holds the accumulators live)
  auto compute_seek = [&](auto Cc) __attribute__((always_inline)) {
    for (; c_pos < x_n; c_pos += S) {
      ct = tile_desc<BM, BN, GMD, B2>(p, x_lo + c_pos);
      c_nk = slices(ct);
      c_ks = 0;
      if (c_nk > 0) break;
      if constexpr (decltype(Cc)::value) store_block(ct);  // a tile without K slices is zero
    }
  };
  // after a step: true while slices are left
  auto advance = [&](auto Cc) __attribute__((always_inline)) -> bool {
    if (++c_ks < c_nk) return true;
    if constexpr (decltype(Cc)::value) {
      store_block(ct);
      zero_acc();
    }
    c_pos += S;
    compute_seek(Cc);
    return c_pos < x_n;
  };

  // The two roles run separate loops (so that neither keeps the other's
  // registers live) with one barrier per K slice each.  Step g: producers
  // send the loads of slice g+PD into register stage g mod PD and write
  // slice g+1 (stage (g+1) mod PD) into LDS buffer (g+1) mod 2; compute waves
  // multiply slice g from buffer g mod 2 and, after a tile's last slice,
  // write the tile out.
  if (producer) {
    load_seek();
    [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
      (issue(std::integral_constant<int, Us>{}, true), ...);
    }(std::make_integer_sequence<int, PD>{});
    compute_seek(std::false_type{});
    if (c_pos >= x_n) return;  // every tile of this workgroup was empty
    LA::store(da[0], smem, ptid);
    LB::store(db[0], smem + BM * BK, ptid);
    __syncthreads();
    int g = 0;
    auto step = [&](auto Vc) __attribute__((always_inline)) -> bool {
      constexpr int V = decltype(Vc)::value;  // g mod (PD * 2 / gcd)
      issue(std::integral_constant<int, V % PD>{}, false);
      if (g + 1 < issued) {
        bf16_t* nxt = smem + ((V + 1) & 1) * BUF;
        LA::store(da[(V + 1) % PD], nxt, ptid);
        LB::store(db[(V + 1) % PD], nxt + BM * BK, ptid);
      }
      __syncthreads();
      ++g;
      return advance(std::false_type{});
    };
    constexpr int UN = (PD % 2 == 0) ? PD : 2 * PD;  // steps until stage and buffer repeat
    while ([&]<int... Vs>(std::integer_sequence<int, Vs...>) __attribute__((always_inline)) {
      return (step(std::integral_constant<int, Vs>{}) && ...);
    }(std::make_integer_sequence<int, UN>{})) {
    }
  } else {
    zero_acc();
    compute_seek(std::true_type{});
    if (c_pos >= x_n) return;
    __syncthreads();
    int g = 0;
    auto step = [&](auto Uc) __attribute__((always_inline)) -> bool {
      constexpr int U = decltype(Uc)::value;
      mma_slice<BM, BN, WGM, WGN, AM, BMD, B2, true, GMD == G_MROWS>(acc, smem + U * BUF, wm, wn,
                                                                     lane, ct.m_hi - ct.m_lo);
      __syncthreads();
      ++g;
      return advance(std::true_type{});
    };
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
  }
}

// Plain-store epilogue of one wave's (32 FM) x 64 block: rows [mb, mb + 32 FM)
// (rows from m_hi on are dropped), columns [nb, nb + 64) (columns from N on
// are dropped), through the wave's own 16 x 64 LDS area `stage`, 16 rows at a
// time: accumulators -> stage (chunk c of row r at c ^ (r mod 8)) -> whole
// 16-byte chunks to memory with buffer stores (a masked lane gets an
// out-of-range offset).  The area is the wave's alone: no workgroup barrier.
template <int FM, int FN, int CPOL>
__device__ __forceinline__ void store_wave_block(const GemmParams& p, f32x16 (&acc)[FM][FN],
                                                 bf16_t* stage, bf16_t* C0, bf16_t* C1, int mb,
                                                 int m_hi, int nb, int lane) {
  constexpr int WTM = 32 * FM, WTN = 32 * FN;
  constexpr int SR = 16;         // staged rows per pass
  constexpr int SCPR = WTN / 8;  // 16-byte chunks per staged row
  static_assert(SCPR == 8, "64-column blocks");
  const int half = lane >> 5;
  const BlockOut bo(p, C0, C1, (int64_t)mb * p.ldc, nb, nb + WTN);
#pragma unroll
  for (int ps = 0; ps < WTM / SR; ++ps) {
    constexpr int PPB = 32 / SR;  // passes per 32-row accumulator block
    const int i = ps / PPB;
    const int rs = (lane & 31) - (ps % PPB) * SR;  // the lane's row in this pass
    if (rs >= 0 && rs < SR) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = j * 32 + 8 * q + 4 * half;
          const int c = (n >> 3) ^ (rs & 7);
          *reinterpret_cast<uint2*>(stage + rs * WTN + c * 8 + (n & 7)) =
              make_uint2(pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                         pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
    }
    // the wave's own LDS writes and reads execute in order; keep the
    // compiler from moving reads above writes (or the next pass's writes
    // above this pass's reads)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    constexpr int NQ = SR * SCPR / 64;  // chunks per lane and pass
    uint4 v[NQ];
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      const int q = h * 64 + lane, r = q / SCPR, c = q % SCPR;
      v[h] = *reinterpret_cast<const uint4*>(stage + r * WTN + (c ^ (r & 7)) * 8);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      const int q = h * 64 + lane, r = ps * SR + q / SCPR, c = q % SCPR;
      const int n = nb + c * 8;
      bo.store<CPOL>(p, v[h], r, n, mb + r < m_hi && n < p.N);
    }
  }
}

// The same for one wave's 32 x 64 block in a single pass through a 32 x 64
// LDS area (4 KB).  Every lane writes its accumulators: row r = lane mod 32,
// 8-byte half h = lane / 32 of 16-byte chunk c.  The chunk sits at physical
// chunk c ^ f(r) of LDS row r, f(r) = (r / 2 mod 4) + 4 (r / 16 mod 2), with
// its two halves swapped in rows with r / 8 odd: the 32 rows' 8-byte pieces
// of one chunk then fall on 64 different banks (row r's LDS row starts at
// bank 32 (r mod 2)).  The readers take whole chunks, 8 lanes per row.
__device__ __forceinline__ int stage32_f(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
template <int CPOL>
__device__ __forceinline__ void store_wave_block32(const GemmParams& p, f32x16 (&acc)[1][2],
                                                   bf16_t* stage, bf16_t* C0, bf16_t* C1, int mb,
                                                   int m_hi, int nb, int lane) {
  const int half = lane >> 5, r = lane & 31;
  const int sw = (r >> 3) & 1;
  const BlockOut bo(p, C0, C1, (int64_t)mb * p.ldc, nb, nb + 64);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * j + q;  // logical chunk: columns 8 c .. 8 c + 7
      *reinterpret_cast<uint2*>(stage + r * 64 + (c ^ stage32_f(r)) * 8 + 4 * (half ^ sw)) =
          make_uint2(pack_bf2(acc[0][j][4 * q], acc[0][j][4 * q + 1]),
                     pack_bf2(acc[0][j][4 * q + 2], acc[0][j][4 * q + 3]));
    }
  // the wave's own LDS writes and reads execute in order; keep the compiler
  // from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = i * 64 + lane, rr = q >> 3, c = q & 7;
    v[i] = swap_halves(*reinterpret_cast<const uint4*>(stage + rr * 64 + (c ^ stage32_f(rr)) * 8),
                       (rr >> 3) & 1);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = i * 64 + lane, rr = q >> 3, c = q & 7;
    const int n = nb + c * 8;
    bo.store<CPOL>(p, v[i], rr, n, mb + rr < m_hi && n < p.N);
  }
}

// ---------------------------------------------------------------------------
// Warp-specialised persistent bf16 GEMM whose producer waves copy the K
// slices straight into LDS (DmaKC / DmaKN) instead of through registers.
// Three slice buffers: at step g the compute waves multiply slice g (buffer
// g mod 3) while the producers send slice g + 2 into the buffer slice g - 1
// has left and then wait for slice g + 1 alone (a vmcnt of one slice's loads:
// loads retire in order), so every slice has two steps to arrive where the
// register-staged form gives it one.  The three buffers take 144 KB of the
// LDS, so the compute waves stage their results 16 rows at a time.  Tile
// order, cursors and the plain-store epilogue's output are those of
// gemm_bf16_ws_kernel; the LDS tiles and the MFMAs are the same, so the
// results are bit-identical.
// ---------------------------------------------------------------------------
// s_waitcnt immediate: vector memory count vm, LDS/scalar count lgkm (15:
// no wait on it).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}
constexpr int vmcnt_imm(int n) { return waitcnt_imm(n, 15); }

template <int BM, int BN, int WGM, int WGN, int NPW, int NB, int AM, int BMD, int GMD, int ROLE>
__global__ __launch_bounds__(64 * (WGM * WGN + NPW)) void gemm_bf16_dma_kernel(GemmParams p) {
  static_assert(NB == 2 || NB == 3, "two or three slice buffers");
  constexpr int NC = WGM * WGN;       // compute waves
  constexpr int NTP = 64 * NPW;       // producer threads
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int BUF = (BM + BN) * BK;
  constexpr int SCPR = WTN / 8;       // 16-byte chunks per staged row
  static_assert(SCPR == 8 && WTM % 32 == 0, "wave blocks of 64 columns");
  static_assert(NB * BUF * 2 + NC * 16 * WTN * 2 <= 160 * 1024, "LDS");
  constexpr int SR = 16;              // staged rows per pass
  constexpr int WST = SR * WTN;       // staging elements per compute wave
  __shared__ __attribute__((aligned(16))) bf16_t smem[NB * BUF + NC * WST];
  typedef DmaLoaders<BM, BN, NTP, AM, BMD, GMD, gathers_a(ROLE)> DL;
  typedef typename DL::LA LA;
  typedef typename DL::LB LB;
  constexpr int L = DL::LOADS;
  static_assert(L * (NB - 2) <= 63, "a slice's loads within the vmcnt range");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= NC;
  const int wm = wave / WGN, wn = wave % WGN;  // compute waves only
  const int ptid = tid - NC * 64;              // producer waves only

  const int count = tile_count<GMD>(p);
  const int xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD, S = gridDim.x / NXCD;
  int x_lo, x_n;
  xcd_tile_range<GMD>(p, count, xcd, x_lo, x_n);
  if (slot >= x_n) return;
  auto slices = [](const TileDesc& t) { return (t.k_hi - t.k_lo + BK - 1) / BK; };

  // ---- producer state: loaders and load cursor
  LA la;
  LB lb;
  int l_pos = slot, l_ks = 0, l_nk = 0;
  auto load_seek = [&]() __attribute__((always_inline)) {
    for (; l_pos < x_n; l_pos += S) {
      const TileDesc t = tile_desc<BM, BN, GMD, B2_NONE>(p, x_lo + l_pos);
      const int nk = slices(t);
      if (nk > 0) {
        l_nk = nk;
        l_ks = 0;
        init_loaders<GMD, B2_NONE>(p, t, la, lb, ptid);
        break;
      }
    }
  };
  // The next slice into buffer `buf`.  Past the last slice the loaders'
  // last state is sent again (a K offset past its range: zeros into a
  // buffer nobody reads), so every step sends the same number of loads.
  auto issue = [&](int buf) __attribute__((always_inline)) {
    la.issue(smem + buf * BUF, l_ks * BK, ptid);
    lb.issue(smem + buf * BUF + BM * BK, l_ks * BK, ptid);
    if (l_pos < x_n && ++l_ks == l_nk) {
      l_pos += S;
      load_seek();
    }
  };

  // ---- compute state
  f32x16 acc[FM][FN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  bf16_t* stage = smem + NB * BUF + (producer ? 0 : wave) * WST;
  auto store_block = [&](const TileDesc& t) __attribute__((always_inline)) {
    bf16_t* C0 = static_cast<bf16_t*>(p.C0);
    bf16_t* C1 = static_cast<bf16_t*>(p.C1);
    if (GMD == G_KROWS) {
      C0 += (int64_t)t.e * p.c_estride;
      if (C1) C1 += (int64_t)t.e * p.c_estride;
    }
    store_wave_block<FM, FN, GMD == G_KROWS ? MOE_OUT_CPOL : 0>(p, acc, stage, C0, C1,
                                                               t.m_lo + wm * WTM, t.m_hi,
                                                               t.n0 + wn * WTN, lane);
  };

  // ---- compute cursor (every wave keeps it; it decides when the loop ends)
  int c_pos = slot, c_ks = 0, c_nk = 0;
  TileDesc ct;
  auto compute_seek = [&](auto Cc) __attribute__((always_inline)) {
    for (; c_pos < x_n; c_pos += S) {
      ct = tile_desc<BM, BN, GMD, B2_NONE>(p, x_lo + c_pos);
      c_nk = slices(ct);
      c_ks = 0;
      if (c_nk > 0) break;
      if constexpr (decltype(Cc)::value) store_block(ct);  // a tile without K slices is zero
    }
  };
  auto advance = [&](auto Cc) __attribute__((always_inline)) -> bool {
    if (++c_ks < c_nk) return true;
    if constexpr (decltype(Cc)::value) {
      store_block(ct);
      zero_acc();
    }
    c_pos += S;
    compute_seek(Cc);
    return c_pos < x_n;
  };

  if (producer) {
    load_seek();
    compute_seek(std::false_type{});
    if (c_pos >= x_n) return;  // every tile of this workgroup was empty
    // slices 0 .. NB-2 go out; slice 0 lands before the first step
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) issue(b);
    // The producers meet the compute waves' barriers with a bare s_barrier:
    // their only writes are the copies into LDS, and the explicit vmcnt wait
    // before it is what makes a slice visible (a workgroup fence would wait
    // for every copy in flight, the next slice's too).
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(L * (NB - 2)));
    __builtin_amdgcn_s_barrier();
    // step g: slice g + NB - 1 into buffer (g - 1) mod NB, then wait for
    // slice g + 1 (the buffer index is a runtime value: one set of address
    // registers for all buffers)
    int fill = NB - 1;
    do {
      issue(fill);
      fill = fill == NB - 1 ? 0 : fill + 1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(L * (NB - 2)));  // slice g + 1 has landed
      __builtin_amdgcn_s_barrier();
    } while (advance(std::false_type{}));
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no copy into LDS outlives the workgroup
  } else {
    zero_acc();
    compute_seek(std::true_type{});
    if (c_pos >= x_n) return;
    __syncthreads();
    int use = 0;  // buffer of slice g
    do {
      mma_slice<BM, BN, WGM, WGN, AM, BMD, B2_NONE, true, GMD == G_MROWS>(acc, smem + use * BUF, wm,
                                                                         wn, lane, ct.m_hi - ct.m_lo);
      use = use == NB - 1 ? 0 : use + 1;
      __syncthreads();
    } while (advance(std::true_type{}));
  }
}

// ---------------------------------------------------------------------------
// Weight gradients of experts with at most STRIP_K rows ("strip" kernel).
// C_e = A_e^T B_e sums over expert e's rows only, and with K <= 256 one
// workgroup holds all of them.  A workgroup per (expert, 256-row block of
// C_e, part of its columns) reads its A block (those 256 rows of C by the
// expert's K rows) once, into its waves' registers (through the LDS, read
// back transposed), then streams the expert's B rows through the LDS one
// 64-deep slice of a 128-column tile at a time and writes the block's
// 256 x 128 output tiles along the row of C_e.  A crosses from L2 into a CU
// once per block of C rows instead of once per output tile: at K = 256 a
// 64 KB output tile costs its 64 KB of B plus a share of 128 KB of A spread
// over the whole row, where the tile kernels read 192 KB for it.  Eight
// 16 KB LDS buffers: in the first steps each holds one 64-deep K slice of
// one half (128 rows of C) of the A block; then two tiles of B, the next one
// sent slice by slice while the current one is multiplied, with one
// workgroup barrier per tile.  Eight waves, two per SIMD, each own 32 rows of
// the block (their A: 64 registers) and all 128 columns of a tile, send the
// copies themselves and stage their results 32 rows at a time.  Every
// 32 x 32 output block takes its MFMAs in the tile kernels' order (K steps of
// 16 in order), so the results are the same bits.  The tile-table launch
// decides on the device which experts are the strip kernel's (zero K cost).
//
// The copies into the LDS are issued as inline assembly, which the compiler
// does not track, and each tile waits for its copies with an explicit vmcnt:
// the compiler, tracking them, waited for every copy in flight before some
// LDS reads.  A lane's vector memory operations complete in the order they
// were issued (copies and stores alike), so tile t has landed once at most
// the operations issued after its copies are outstanding: the stores of tile
// t - 1.  The wait counts take the fewest stores a tile can issue (a count
// too small only waits longer).
// ---------------------------------------------------------------------------
constexpr int STRIP_M = 256;  // output rows per workgroup
constexpr int STRIP_N = 128;  // columns of a B tile
static_assert(STRIP_K >= 0 && STRIP_K <= 4 * BK, "the strip kernel holds at most four K slices");
// Cache policy of the strip kernel's result stores: non-temporal for the
// gate/up gradient, sc1 for the down projection's (measured: the down
// gradient 146-149 vs 165-167 us and the gate/up gradient, which runs two
// kernels later, 247-252 vs 267-270 us, the down input gradient in between
// 8 us slower; sc1 for the gate/up gradient made it slower).
#ifndef MOE_STRIP_DOWN_CPOL
#define MOE_STRIP_DOWN_CPOL 16
#endif

// Buffer descriptor words over 2^31 - 1 bytes from `base` (as make_rsrc).
__device__ __forceinline__ u32x4 rsrc_words(const void* base) {
  const uint64_t a = (uint64_t)base;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, 0x7fffffffu, 0x00020000u};
}
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t*)p;
}
// 16 bytes per lane from the buffer (byte offset voff; out of range: zeros)
// into the LDS at lds_byte + 16 lane, untracked by the compiler.  No output
// registers; the caller waits for the copy with vmcnt.
__device__ __forceinline__ void dma16_untracked(u32x4 r, uint32_t lds_byte, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_byte), "v"(voff), "s"(r)
      : "memory", "m0");
}

// GDY (the down projection's gradient with dYp never written): B row k is
// row a_rows[k] of dY and A row k is scaled by the row's gate weight once, in
// the registers (bf16, round to nearest even).
template <bool GDY, int ROLE>
__global__ __launch_bounds__(512) void gemm_bf16_strip_kernel(GemmParams p) {
  static_assert(!GDY || ROLE == R_DOWN_WGRAD, "the dY form is the down projection's");
  constexpr bool AG = gathers_a(ROLE);
  constexpr int OCP = ROLE == R_DOWN_WGRAD ? MOE_STRIP_DOWN_CPOL : MOE_OUT_CPOL;
  constexpr int SL = BK * STRIP_N;  // one buffer: [64][128] bf16 (the KN layout)
  __shared__ __attribute__((aligned(16))) bf16_t sbuf[8 * SL];
  __shared__ __attribute__((aligned(16))) bf16_t stage_all[8 * 32 * 64];
  using std::integral_constant;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // rows 32 wave .. + 31 of the block
  // work item (expert e, row block, column part): the columns of C_e are
  // split in `ncs` parts of whole tiles, so that the items fill the CUs
  // evenly
  const int mstrips = (p.M + STRIP_M - 1) / STRIP_M, ncs = p.col_parts;
  const int ntile_all = (p.N + STRIP_N - 1) / STRIP_N;
  const int id = remap_xcd(blockIdx.x, gridDim.x);  // an expert's items on one XCD
  const int e = __builtin_amdgcn_readfirstlane(id / (mstrips * ncs));
  const int rem = id - e * mstrips * ncs;
  const int mblk = __builtin_amdgcn_readfirstlane(rem / ncs);
  const int cpart = __builtin_amdgcn_readfirstlane(rem - mblk * ncs);
  const int m0 = mblk * STRIP_M;
  const int t_first = cpart * ntile_all / ncs;  // the part's tiles [t_first, t_first + ntile)
  const int ntile = (cpart + 1) * ntile_all / ncs - t_first;
  // the strip path is on when the tile-table launch gave every expert zero
  // cost (every expert has at most STRIP_K rows); else the tile kernels run
  // them all
  if (ld_table(p.kcost, e + 1) != ld_table(p.kcost, e)) return;
  const int k_lo = ld_table(p.off, e), k_hi = ld_table(p.off, e + 1);
  const int kn = k_hi - k_lo;
  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B = static_cast<const bf16_t*>(p.B0);
  // lane chunk q = tid + 512 i of a buffer: row q / 16 of the slice, logical
  // 16-byte chunk (q mod 16) ^ ((row mod 4) * 4) (kn_swz inverted)
  int crow[2], ccol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 512 * i;
    crow[i] = q >> 4;
    ccol[i] = ((q & 15) ^ ((crow[i] & 3) << 2)) * 8;
  }
  const uint32_t lds0 = lds_addr(sbuf) + 64 * wave * 16;  // the wave's first chunk in buffer 0

  // ---- A: K slice s, C rows m0 + 128 h .. + 127 into buffer 2 s + h (the
  // gather roles find row k's source row in the row table)
  {
    const u32x4 ra = rsrc_words(AG ? A : A + (int64_t)k_lo * p.lda);
    int vo[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = s * BK + crow[i];
        int64_t row = k;
        if constexpr (AG) row = kn > 0 ? p.a_rows[min(k_lo + k, k_hi - 1)] : 0;
        vo[s][i] = k < kn ? (int)((row * p.lda + m0 + ccol[i]) * 2) : OOB;
      }
#pragma unroll
    for (int bi = 0; bi < 8; ++bi)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int h = bi & 1;
        const bool ok = vo[bi >> 1][i] != OOB && m0 + h * STRIP_N + ccol[i] < p.M;
        dma16_untracked(ra, lds0 + (bi * SL + 512 * i * 8) * 2, ok ? vo[bi >> 1][i] + h * STRIP_N * 2 : OOB);
      }
  }
  // GDY: the K rows' gate weights and dY rows (byte offsets of the lane's
  // chunks' rows, OOB past the expert's rows)
  float* gs = reinterpret_cast<float*>(stage_all);
  int bro[4][2];
  if constexpr (GDY) {
    if (tid < 4 * BK) gs[tid] = tid < kn ? p.row_gate[p.row_slot[k_lo + tid]] : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int k = s * BK + crow[i];
        const int64_t row = kn > 0 ? p.a_rows[min(k_lo + k, k_hi - 1)] : 0;
        bro[s][i] = k < kn ? (int)(row * p.ldb * 2) : OOB;
      }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  __syncthreads();
  bf16x8 af[16];  // the wave's 32 rows of A over K, one fragment per K step of 16
  {
    const int h = wave >> 2, mb = (wave & 3) * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[4 * s + ks] = frag_kn<STRIP_N>(sbuf + (2 * s + h) * SL, mb, ks, lane);
    if constexpr (GDY) {
      // the fragment of K step ks holds rows 16 ks + 8 (lane / 32) + 0..7
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const float4 g0 = *reinterpret_cast<const float4*>(gs + 16 * ks + 8 * (lane >> 5));
        const float4 g1 = *reinterpret_cast<const float4*>(gs + 16 * ks + 8 * (lane >> 5) + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) af[ks][j] = (__bf16)((float)af[ks][j] * gv[j]);
      }
    }
  }
  __syncthreads();  // every wave has its A before B overwrites the buffers

  // ---- B: tile t's K slice s into buffer 4 (t mod 2) + s; tiles from
  // `ntile` on (the pad to an even count, and the sends past the last tile)
  // read nothing
  auto col_tile = [&](int t) { return t < ntile ? t_first + t : ntile_all; };
  int bo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) bo[i] = (int)(((int64_t)crow[i] * p.ldb + ccol[i]) * 2);
  auto send_b = [&](int bi, int t, int s) __attribute__((always_inline)) {
    const u32x4 rb = rsrc_words(GDY ? B : B + (int64_t)(k_lo + s * BK) * p.ldb);
    const int c = col_tile(t);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool ok = s * BK + crow[i] < kn && c * STRIP_N + ccol[i] < p.N;
      const int o = GDY ? bro[s][i] + (c * STRIP_N + ccol[i]) * 2 : bo[i] + c * STRIP_N * 2;
      dma16_untracked(rb, lds0 + (bi * SL + 512 * i * 8) * 2, ok ? o : OOB);
    }
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) send_b(j, 0, j);

  bf16_t* C0 = static_cast<bf16_t*>(p.C0) + (int64_t)e * p.c_estride;
  bf16_t* C1 = p.C1 ? static_cast<bf16_t*>(p.C1) + (int64_t)e * p.c_estride : nullptr;
  bf16_t* stage = stage_all + wave * 32 * 64;
  f32x16 acc[2][1][2];  // [64-column half of the tile][32-row block][32-column block]
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[h][0][j][r] = 0.f;
  };
  zero_acc();

  // Tile t (its slices in buffers 4 h .. 4 h + 3, h = t mod 2).  Its copies
  // went out during tile t - 1 (tile 0's before the loop); issued after them:
  // the stores of tile t - 1 (8 per lane at least).
  auto tile = [&](auto Hc, auto Fc, int t) __attribute__((always_inline)) {
    constexpr int h = decltype(Hc)::value;
    constexpr bool first = decltype(Fc)::value;
    // this lane's copies of the tile have landed and its reads of the last
    // tile are done; then every wave's
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(first && h == 0 ? 0 : 8, 0));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // slice s of tile t + 1 into the buffer tile t - 1's slice s has left,
      // one slice per slice of MFMAs (a wave whose copies wait for room in
      // the memory pipeline stalls at the copy, not at all four)
      send_b(4 * (1 - h) + s, t + 1, s);
      const bf16_t* bs = sbuf + (4 * h + s) * SL;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bfr[j] = frag_kn<STRIP_N>(bs, 32 * j, ks, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j >> 1][0][j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              bfr[j], af[4 * s + ks], acc[j >> 1][0][j & 1], 0, 0, 0);
      }
    }
    const int n0 = col_tile(t) * STRIP_N;
    store_wave_block32<OCP>(p, acc[0], stage, C0, C1, m0 + wave * 32, p.M, n0, lane);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the first half's reads are done
    store_wave_block32<OCP>(p, acc[1], stage, C0, C1, m0 + wave * 32, p.M, n0 + 64, lane);
    zero_acc();
  };
  tile(integral_constant<int, 0>{}, std::true_type{}, 0);
  tile(integral_constant<int, 1>{}, std::true_type{}, 1);
  for (int t0 = 2; t0 < ntile; t0 += 2) {
    tile(integral_constant<int, 0>{}, std::false_type{}, t0);
    tile(integral_constant<int, 1>{}, std::false_type{}, t0 + 1);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // no copy into LDS outlives the workgroup
}

// ---------------------------------------------------------------------------
// fp32 kernel: one output (or one gate/up pair) per thread, fp32 FMA.
// ---------------------------------------------------------------------------
template <int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  const int n = blockIdx.x * 16 + (threadIdx.x & 15);
  const int m = blockIdx.y * 16 + (threadIdx.x >> 4);
  const float* A = static_cast<const float*>(p.A);
  const float* B0 = static_cast<const float*>(p.B0);
  const float* B1 = static_cast<const float*>(p.B1);
  int e = 0, k_lo = 0, k_hi = p.K;
  const int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? p.I : p.N;
  if (n >= ncols) return;
  if (GMD == G_MROWS) {
    if (m >= p.off[p.groups]) return;
    int lo = 0, hi = p.groups - 1;  // last e with off[e] <= m
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (p.off[mid] <= m) lo = mid; else hi = mid - 1;
    }
    e = lo;
    B0 += (int64_t)e * p.b_estride;
    if (B2 != B2_NONE) B1 += (int64_t)e * p.b_estride;
  } else {
    if (m >= p.M) return;
    if (GMD == G_KROWS) {
      e = blockIdx.z;
      if (p.off) { k_lo = p.off[e]; k_hi = p.off[e + 1]; }
      else if (p.k_chunk > 0) { k_lo = min(p.K, e * p.k_chunk); k_hi = min(p.K, k_lo + p.k_chunk); }
    }
  }
  // gather roles: logical A row j is row a_rows[j] / a_rows_div
  auto a_row = [&](int j) -> int64_t {
    return gathers_a(ROLE) ? (int64_t)((uint32_t)p.a_rows[j] / (uint32_t)p.a_rows_div) : j;
  };
  auto a_at = [&](int k) -> float {
    return AM == A_KC ? A[a_row(m) * p.lda + k] : A[a_row(k) * p.lda + m];
  };
  auto b_at = [&](const float* B, int k, int col) -> float {
    return BMD == B_NC ? B[(int64_t)k * p.ldb + col] : B[(int64_t)col * p.ldb + k];
  };
  float acc = 0.f, acc2 = 0.f;
  for (int k = k_lo; k < k_hi; ++k) {
    float a = a_at(k);
    if (B2 == B2_NHALF) {
      acc = fmaf(a, b_at(B0, k, n), acc);
      acc2 = fmaf(a, b_at(B1, k, n), acc2);
    } else if (B2 == B2_KSPLIT) {
      acc = fmaf(a, k < p.k_split ? b_at(B0, k, n) : b_at(B1, k - p.k_split, n), acc);
    } else {
      acc = fmaf(a, b_at(B0, k, n), acc);
    }
  }
  if constexpr (EPI == EPI_STORE) {
    float* C = static_cast<float*>(p.C0);
    int nn = n;
    if (p.n_split > 0 && nn >= p.n_split) { C = static_cast<float*>(p.C1); nn -= p.n_split; }
    if (GMD == G_KROWS) C += (int64_t)e * p.c_estride;
    C[(int64_t)m * p.ldc + nn] = acc;
  } else if constexpr (EPI == EPI_ACCUM) {
    static_cast<float*>(p.C0)[(int64_t)m * p.ldc + n] += acc;
  } else if constexpr (EPI == EPI_F32_BIAS) {
    static_cast<float*>(p.C0)[(GMD == G_KROWS ? (int64_t)e * p.c_estride : 0) + (int64_t)m * p.ldc + n] =
        acc + (p.bias ? p.bias[n] : 0.f);
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int64_t I = p.I;
    float* H = static_cast<float*>(p.C0);
    if (H) { H[m * 2 * I + n] = acc; H[m * 2 * I + I + n] = acc2; }
    static_cast<float*>(p.C2)[m * I + n] = acc / (1.0f + expf(-acc)) * acc2;
  } else if constexpr (EPI == EPI_DSWIGLU) {
    const int64_t I = p.I;
    const float* H = static_cast<const float*>(p.aux);
    float g = H[m * 2 * I + n], u = H[m * 2 * I + I + n];
    float sg = 1.0f / (1.0f + expf(-g));
    float* dH = static_cast<float*>(p.C0);
    dH[m * 2 * I + n] = acc * u * sg * (1.0f + g * (1.0f - sg));
    dH[m * 2 * I + I + n] = acc * g * sg;
  }
}

// ---------------------------------------------------------------------------
// Tile table for row-grouped GEMMs.
// ---------------------------------------------------------------------------
// Workgroup 0 builds the table for 256-row tiles, workgroup 1 the one for
// 128-row tiles.
// Workgroups 3 .. 3 + ntok - 1 (launched with a token table only) write the
// token rows of the routed rows; the workgroups after them (launched with a
// CombinePrep only) prepare the fused combine, one wavefront per token.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* off, int groups,
                                                          int32_t* tiles256, int32_t* tiles128,
                                                          int32_t* kcost, const int32_t* perm,
                                                          int k, int32_t* tok, int ntok,
                                                          CombinePrep cmb) {
  if (blockIdx.x >= 3 + ntok) {  // one wavefront per token
    const int lane = threadIdx.x & 63;
    const int t = (blockIdx.x - 3 - ntok) * 16 + (threadIdx.x >> 6);
    if (t >= cmb.T) return;
    const bool kept_j = lane < cmb.k && cmb.inv[(int64_t)t * cmb.k + lane] >= 0;
    const int kept = __popcll(__ballot(kept_j));
    if (lane == 0) cmb.kept[t] = kept;
    for (int c = lane; c < cmb.ncb; c += 64) cmb.cnt[(int64_t)t * cmb.ncb + c] = 0;
    if (kept == 0) {
      uint4* y = reinterpret_cast<uint4*>(static_cast<char*>(cmb.y) + (int64_t)t * cmb.y_row_bytes);
      for (int c = lane; c < cmb.y_row_bytes / 16; c += 64) y[c] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  if (blockIdx.x >= 3) {
    const int R = off[groups];
    for (int p = (blockIdx.x - 3) * 1024 + threadIdx.x; p < R; p += ntok * 1024)
      tok[p] = (int)((uint32_t)perm[p] / (uint32_t)k);
    return;
  }
  const bool cost = blockIdx.x == 2;  // workgroup 2: the weight-gradient cost prefix
  if (cost && kcost == nullptr) return;
  const int bm = blockIdx.x == 0 ? 256 : 128;
  int32_t* tiles = blockIdx.x == 0 ? tiles256 : tiles128;
  __shared__ int32_t scan[1024];
  __shared__ int32_t carry;
  __shared__ int32_t strip_all;  // every expert fits the strip kernel (cost workgroup)
  if (threadIdx.x == 0) {
    carry = 0;
    strip_all = STRIP_K > 0;
  }
  __syncthreads();
  if (cost && STRIP_K > 0) {
    bool big = false;
    for (int e = threadIdx.x; e < groups; e += 1024) big |= off[e + 1] - off[e] > STRIP_K;
    if (big) strip_all = 0;  // benign race: every writer stores 0
    __syncthreads();
  }
  for (int base = 0; base < groups; base += 1024) {
    int e = base + threadIdx.x;
    int cnt = 0, o = 0;
    if (e < groups) {
      o = off[e];
      const int rows = off[e + 1] - o;
      cnt = !cost ? (rows + bm - 1) / bm : strip_all ? 0 : (rows + BK - 1) / BK + KCOST_FIXED;
    }
    scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {  // inclusive Hillis-Steele scan
      int v = threadIdx.x >= s ? scan[threadIdx.x - s] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    int first = carry + scan[threadIdx.x] - cnt;
    if (cost) {
      if (e < groups) kcost[e + 1] = first + cnt;
    } else {
      for (int t = 0; t < cnt; ++t) {
        tiles[1 + 2 * (first + t)] = e;
        tiles[2 + 2 * (first + t)] = o + t * bm;
      }
    }
    __syncthreads();
    if (threadIdx.x == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (cost) kcost[0] = 0;
    else tiles[0] = carry;
  }
}

moe_status_t launch_tile_tables(const int32_t* off, int groups, int32_t* tiles256,
                                int32_t* tiles128, int32_t* kcost, hipStream_t s,
                                const int32_t* perm, int k, int32_t* tok, int rows_cap,
                                const CombinePrep* cmb) {
  ProfScope prof("tile_table", s);
  const int ntok =
      perm ? (int)std::min<int64_t>(64, std::max<int64_t>(1, ceil_div(rows_cap, 1024))) : 0;
  const int ncmb = cmb ? (int)ceil_div(cmb->T, 16) : 0;  // 16 tokens per workgroup
  const CombinePrep none{};
  tile_table_kernel<<<3 + ntok + ncmb, 1024, 0, s>>>(off, groups, tiles256, tiles128, kcost, perm,
                                                     k, tok, ntok, cmb ? *cmb : none);
  return check_launch("tile_table_kernel");
}

int tile_bm(TileCfg cfg) {
  return cfg == TILE_64x64 ? 64 : (cfg == TILE_128x128 || cfg == TILE_128x256) ? 128 : 256;
}
int tile_bn(TileCfg cfg) {
  return (cfg == TILE_256x256 || cfg == TILE_128x256) ? 256
         : (cfg == TILE_256x128 || cfg == TILE_128x128) ? 128
                                                         : 64;
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------
// Tile shape of each expert GEMM (build-time tunable).
#ifndef MOE_TILE_GATEUP_FWD
#define MOE_TILE_GATEUP_FWD TILE_256x256
#endif
#ifndef MOE_TILE_DOWN_FWD
#define MOE_TILE_DOWN_FWD TILE_128x256
#endif
#ifndef MOE_TILE_DOWN_DGRAD
#define MOE_TILE_DOWN_DGRAD TILE_256x128
#endif
#ifndef MOE_TILE_GATEUP_DGRAD
#define MOE_TILE_GATEUP_DGRAD TILE_256x256
#endif
#ifndef MOE_WGRAD_TILE
#define MOE_WGRAD_TILE TILE_256x128
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 2
#endif
#ifndef MOE_WIDE_WAVES
#define MOE_WIDE_WAVES 8
#endif

// role, name, tile, A layout, B layout, grouping, two-source B, epilogue
#define MOE_GEMM_ROLES(X)                                                                          \
  X(R_ROUTE_LOGITS, "route_logits", TILE_64x64, A_KC, B_NC, G_DENSE, B2_NONE, EPI_F32_BIAS)        \
  X(R_GATEUP_FWD, "ffn_gateup_fwd", MOE_TILE_GATEUP_FWD, A_KC, B_NC, G_MROWS, B2_NHALF, EPI_SWIGLU) \
  X(R_DOWN_FWD, "ffn_down_fwd", MOE_TILE_DOWN_FWD, A_KC, B_NC, G_MROWS, B2_NONE, EPI_STORE)         \
  X(R_DOWN_DGRAD, "ffn_down_dgrad", MOE_TILE_DOWN_DGRAD, A_KC, B_KC, G_MROWS, B2_NONE, EPI_DSWIGLU) \
  X(R_GATEUP_DGRAD, "ffn_gateup_dgrad", MOE_TILE_GATEUP_DGRAD, A_KC, B_KC, G_MROWS, B2_KSPLIT,      \
    EPI_STORE)                                                                                     \
  X(R_DOWN_WGRAD, "ffn_down_wgrad", MOE_WGRAD_TILE, A_MC, B_NC, G_KROWS, B2_NONE, EPI_STORE)        \
  X(R_GATEUP_WGRAD, "ffn_gateup_wgrad", MOE_WGRAD_TILE, A_MC, B_NC, G_KROWS, B2_NONE, EPI_STORE)    \
  X(R_ROUTE_DW, "route_bwd_dw", TILE_64x64, A_MC, B_NC, G_KROWS, B2_NONE, EPI_F32_BIAS)            \
  X(R_ROUTE_DX, "route_bwd_dx", TILE_64x64, A_KC, B_KC, G_DENSE, B2_NONE, EPI_ACCUM)                \
  X(R_GATEUP_FWD_GATHER, "ffn_gateup_fwd_gather", MOE_TILE_GATEUP_FWD, A_KC, B_NC, G_MROWS, B2_NHALF, \
    EPI_SWIGLU)                                                                                    \
  X(R_GATEUP_WGRAD_GATHER, "ffn_gateup_wgrad_gather", MOE_WGRAD_TILE, A_MC, B_NC, G_KROWS, B2_NONE, \
    EPI_STORE)                                                                                     \
  X(R_DOWN_FWD_COMBINE, "ffn_down_fwd_combine", MOE_TILE_DOWN_FWD, A_KC, B_NC, G_MROWS, B2_NONE,    \
    EPI_STORE)                                                                                     \
  X(R_DOWN_DGRAD_GATHER, "ffn_down_dgrad_dy", MOE_TILE_DOWN_DGRAD, A_KC, B_KC, G_MROWS, B2_NONE,    \
    EPI_DSWIGLU)

// A role may take a second tile shape when its N (output columns) is large:
// role, tile, smallest N (build-time tunable).
// (down dgrad: the 256x256 tile from N = 768 on; at N = 768 it reads the dYp
// rows three times instead of six)
#ifndef MOE_DOWN_DGRAD_WIDE_N
#define MOE_DOWN_DGRAD_WIDE_N 768
#endif
#define MOE_GEMM_ALT_TILES(X)                              \
  X(R_DOWN_DGRAD, TILE_256x256, MOE_DOWN_DGRAD_WIDE_N) \
  X(R_DOWN_DGRAD_GATHER, TILE_256x256, MOE_DOWN_DGRAD_WIDE_N)

constexpr int role_alt_tile(GemmRole role) {
#define X(r, t, nmin) \
  if (role == r) return t;
  MOE_GEMM_ALT_TILES(X)
#undef X
  return -1;
}

TileCfg role_tile(GemmRole role, int n) {
#define X(r, t, nmin) \
  if (role == r && n >= nmin) return t;
  MOE_GEMM_ALT_TILES(X)
#undef X
  switch (role) {
#define X(r, n, t, a, b, g, t2, e) \
  case r: return t;
    MOE_GEMM_ROLES(X)
#undef X
  }
  return TILE_64x64;
}

const char* role_name(GemmRole role) {
  switch (role) {
#define X(r, n, t, a, b, g, t2, e) \
  case r: return n;
    MOE_GEMM_ROLES(X)
#undef X
  }
  return "gemm";
}

template <int CFG> struct TileDims;
template <> struct TileDims<TILE_256x256> { static constexpr int BM = 256, BN = 256; };
template <> struct TileDims<TILE_256x128> { static constexpr int BM = 256, BN = 128; };
template <> struct TileDims<TILE_128x128> { static constexpr int BM = 128, BN = 128; };
template <> struct TileDims<TILE_64x64> { static constexpr int BM = 64, BN = 64; };
template <> struct TileDims<TILE_128x256> { static constexpr int BM = 128, BN = 256; };

// Roles that run the warp-specialised kernel, and roles that run the
// persistent kernel (bit r = role r; build-time tunable).
#ifndef MOE_WS_ROLES
#define MOE_WS_ROLES \
  ((1 << R_DOWN_FWD) | (1 << R_DOWN_WGRAD) | (1 << R_GATEUP_WGRAD) | (1 << R_GATEUP_WGRAD_GATHER) | \
   (1 << R_DOWN_FWD_COMBINE))
#endif
#ifndef MOE_PERSIST_ROLES
#define MOE_PERSIST_ROLES 0
#endif
// Warp-specialised roles whose producers copy K slices straight into LDS
// (build-time tunable; the fused combine keeps the register-staged form).
#ifndef MOE_DMA_WAVE_ROWS
#define MOE_DMA_WAVE_ROWS 64
#endif
#ifndef MOE_DMA_ROLES
#define MOE_DMA_ROLES \
  ((1 << R_DOWN_FWD) | (1 << R_DOWN_WGRAD) | (1 << R_GATEUP_WGRAD) | (1 << R_GATEUP_WGRAD_GATHER))
#endif
// Register stages of the warp-specialised kernel's producer waves; its
// compute waves each own a 64 x 64 block of the tile.
#ifndef MOE_WS_STAGES
#define MOE_WS_STAGES 2
#endif
#ifndef MOE_WS_WAVE_ROWS
#define MOE_WS_WAVE_ROWS 64
#endif
#ifndef MOE_WS_PRODUCER_WAVES
#define MOE_WS_PRODUCER_WAVES 4
#endif

// Compute units of the current device (queried once per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Workgroups of a persistent launch: as many as fit on the device at once,
// at most one per tile, a multiple of the XCD count.
static int persistent_grid(int occupancy, int max_tiles) {
  int64_t g = std::min<int64_t>((int64_t)std::max(occupancy, 1) * device_cus(), max_tiles);
  return (int)std::max<int64_t>(NXCD, g / NXCD * NXCD);
}

template <int CFG, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
static void launch_bf16(const GemmParams& p, int grid, hipStream_t s) {
  constexpr int BMt = TileDims<CFG>::BM, BNt = TileDims<CFG>::BN;
  constexpr int P = (BMt >= 128) ? MOE_GEMM_STAGES : 2;  // register stages in flight
  // 256x256 tiles: MOE_WIDE_WAVES = 8 runs two waves per SIMD (2 x 4 grid)
  constexpr int WGN = (BMt == 256 && BNt == 256 && MOE_WIDE_WAVES == 8) ? 4 : 2;
  constexpr int NT = 64 * 2 * WGN;
  if constexpr (((MOE_DMA_ROLES >> ROLE) & 1) && EPI == EPI_STORE && B2 == B2_NONE &&
                ROLE != R_DOWN_FWD_COMBINE) {
    // compute waves with MOE_DMA_WAVE_ROWS x 64 blocks; three slice buffers
    // while they fit in the LDS, else two
    constexpr int CWM = BMt / MOE_DMA_WAVE_ROWS, CWN = BNt / 64;
    constexpr int NBUF = 3 * (BMt + BNt) * BK * 2 + CWM * CWN * 16 * 64 * 2 <= 160 * 1024 ? 3 : 2;
    constexpr int WS_NT = 64 * (CWM * CWN + MOE_WS_PRODUCER_WAVES);
    const auto kern =
        gemm_bf16_dma_kernel<BMt, BNt, CWM, CWN, MOE_WS_PRODUCER_WAVES, NBUF, AM, BMD, GMD, ROLE>;
    static int occupancy = 0;
    if (occupancy <= 0 &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occupancy, kern, WS_NT, 0) != hipSuccess)
      occupancy = 1;
    kern<<<persistent_grid(occupancy, grid), WS_NT, 0, s>>>(p);
  } else if constexpr (((MOE_WS_ROLES >> ROLE) & 1) && (EPI != EPI_STORE || B2 != B2_NHALF)) {
    // compute waves with MOE_WS_WAVE_ROWS x 64 blocks (64 x 64 for the fused
    // combine, whose counters go one row per lane), and the producer waves
    constexpr int WROWS = ROLE == R_DOWN_FWD_COMBINE ? 64 : MOE_WS_WAVE_ROWS;
    constexpr int CWM = BMt / WROWS, CWN = BNt / 64;
    constexpr int WS_NT = 64 * (CWM * CWN + MOE_WS_PRODUCER_WAVES);
    const auto kern = gemm_bf16_ws_kernel<BMt, BNt, CWM, CWN, MOE_WS_PRODUCER_WAVES, MOE_WS_STAGES,
                                          AM, BMD, GMD, B2, EPI, ROLE>;
    static int occupancy = 0;
    if (occupancy <= 0 &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occupancy, kern, WS_NT, 0) != hipSuccess)
      occupancy = 1;
    kern<<<persistent_grid(occupancy, grid), WS_NT, 0, s>>>(p);
  } else if constexpr ((MOE_PERSIST_ROLES >> ROLE) & 1) {
    const auto kern = gemm_bf16_persistent_kernel<BMt, BNt, 2, WGN, AM, BMD, GMD, B2, EPI, ROLE>;
    static int occupancy = 0;  // per kernel instance; the same on every gfx950 device
    if (occupancy <= 0 &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occupancy, kern, NT, 0) != hipSuccess)
      occupancy = 1;
    kern<<<persistent_grid(occupancy, grid), NT, 0, s>>>(p);
  } else {
    gemm_bf16_kernel<BMt, BNt, 2, WGN, P, AM, BMD, GMD, B2, EPI, ROLE><<<grid, NT, 0, s>>>(p);
  }
}

// The role's usual tile, or its alternate tile (ALT >= 0) when `alt`.
template <int ALT, int CFG, int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
static void launch_bf16_role(const GemmParams& p, int grid, hipStream_t s, bool alt) {
  if constexpr (ALT >= 0) {
    if (alt) {
      launch_bf16<ALT, AM, BMD, GMD, B2, EPI, ROLE>(p, grid, s);
      return;
    }
  }
  launch_bf16<CFG, AM, BMD, GMD, B2, EPI, ROLE>(p, grid, s);
}

template <int AM, int BMD, int GMD, int B2, int EPI, int ROLE>
static void launch_f32(const GemmParams& p, int max_rows, hipStream_t s) {
  int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? p.I : p.N;
  dim3 grid((unsigned)ceil_div(ncols, 16), (unsigned)ceil_div(max_rows, 16),
            GMD == G_KROWS ? (unsigned)p.groups : 1u);
  gemm_f32_kernel<AM, BMD, GMD, B2, EPI, ROLE><<<grid, 256, 0, s>>>(p);
}

// Column parts of the strip kernel's work items: the split (1 to 4 parts of
// whole tiles) that moves the fewest bytes through the busiest CU, with every
// expert taken to be the strip kernel's (rounds of one item per CU, each
// reading its A block once and its part of the B tiles).
static int strip_column_parts(const GemmParams& p) {
  const int cus = device_cus();
  const int64_t ntile = ceil_div(p.N, STRIP_N);
  const int64_t items1 = (int64_t)p.groups * ceil_div(p.M, STRIP_M);
  int best = 1;
  int64_t best_cost = -1;
  for (int c = 1; c <= 4 && c <= ntile; ++c) {
    const int64_t rounds = ceil_div(items1 * c, cus);
    const int64_t cost = rounds * (STRIP_M + ceil_div(ntile, c) * STRIP_N);  // A rows + B columns
    if (best_cost < 0 || cost < best_cost) { best = c; best_cost = cost; }
  }
  return best;
}

static moe_status_t launch_gemm_kernels(bool is_bf16, GemmRole role, const GemmParams& p,
                                        int max_m_tiles, hipStream_t s) {
  const char* name = role_name(role);
  if (!is_bf16) {
    if (role == R_DOWN_DGRAD_GATHER) {
      set_error("GEMM %s: bf16 only", name);
      return MOE_ERR_UNSUPPORTED;
    }
    // rows to cover: G_MROWS row capacity (passed as max_m_tiles), else M
    switch (role) {
#define X(r, n, t, a, b, g, t2, e)                        \
  case r: {                                               \
    const int rows = (g == G_MROWS) ? max_m_tiles : p.M;  \
    if (rows <= 0) return MOE_OK;                         \
    launch_f32<a, b, g, t2, e, r>(p, rows, s);            \
    break;                                                \
  }
      MOE_GEMM_ROLES(X)
#undef X
    }
    return check_launch(name);
  }
  // weight gradients: the experts with at most STRIP_K rows in the strip
  // kernel first, then the others in the role's tile kernel
  GemmParams q = p;
  if (STRIP_K > 0 && !p.k_strip && p.off != nullptr && p.kcost != nullptr && p.groups > 0 && p.M > 0 &&
      (role == R_DOWN_WGRAD || role == R_GATEUP_WGRAD || role == R_GATEUP_WGRAD_GATHER)) {
    GemmParams sp = p;
    sp.col_parts = strip_column_parts(p);
    const int64_t grid = (int64_t)p.groups * ceil_div(p.M, STRIP_M) * sp.col_parts;
    if (grid > 0x7fffffff) {
      set_error("GEMM %s: grid too large", name);
      return MOE_ERR_UNSUPPORTED;
    }
    if (role == R_DOWN_WGRAD) gemm_bf16_strip_kernel<false, R_DOWN_WGRAD><<<(int)grid, 512, 0, s>>>(sp);
    else if (role == R_GATEUP_WGRAD)
      gemm_bf16_strip_kernel<false, R_GATEUP_WGRAD><<<(int)grid, 512, 0, s>>>(sp);
    else gemm_bf16_strip_kernel<false, R_GATEUP_WGRAD_GATHER><<<(int)grid, 512, 0, s>>>(sp);
    const moe_status_t st = check_launch(name);
    if (st != MOE_OK) return st;
    q.k_strip = 1;
  }
  switch (role) {
#define X(r, n, t, a, b, g, t2, e)                                                        \
  case r: {                                                                               \
    const int64_t per = (int64_t)max_m_tiles * p.n_tiles;                                 \
    const int64_t grid = (g == G_KROWS) ? per * p.groups : per;                           \
    if (grid <= 0) return MOE_OK;                                                         \
    if (grid > 0x7fffffff) {                                                              \
      set_error("GEMM %s: grid too large", name);                                         \
      return MOE_ERR_UNSUPPORTED;                                                         \
    }                                                                                     \
    launch_bf16_role<role_alt_tile(r), t, a, b, g, t2, e, r>(                               \
        q, (int)grid, s, role_tile(r, p.N) != t);                                          \
    break;                                                                                \
  }
    MOE_GEMM_ROLES(X)
#undef X
  }
  return check_launch(name);
}

moe_status_t launch_gemm(bool is_bf16, GemmRole role, const GemmParams& p, int max_m_tiles,
                         hipStream_t s) {
  ProfScope prof(role_name(role), s);
  return launch_gemm_kernels(is_bf16, role, p, max_m_tiles, s);
}

moe_status_t launch_down_wgrad_dy(const GemmParams& p, const void* dyp, int max_m_tiles,
                                  hipStream_t s) {
  const char* name = "ffn_down_wgrad_dy";
  if (STRIP_K <= 0 || !p.off || !p.kcost || !p.a_rows || !p.row_gate || !p.row_slot || !dyp) {
    set_error("GEMM %s (dY form): needs offsets, K costs, the token table, the gate weights "
              "and dYp, and the strip kernel", name);
    return MOE_ERR_ARG;
  }
  ProfScope prof(name, s);
  if (p.groups <= 0 || p.M <= 0) return MOE_OK;
  GemmParams sp = p;
  sp.col_parts = strip_column_parts(p);
  const int64_t grid = (int64_t)p.groups * ceil_div(p.M, STRIP_M) * sp.col_parts;
  if (grid > 0x7fffffff) {
    set_error("GEMM %s: grid too large", name);
    return MOE_ERR_UNSUPPORTED;
  }
  gemm_bf16_strip_kernel<true, R_DOWN_WGRAD><<<(int)grid, 512, 0, s>>>(sp);
  const moe_status_t st = check_launch(name);
  if (st != MOE_OK) return st;
  // the experts of nonzero K cost (all of them, when one has more than
  // STRIP_K rows) in the tile kernel, on dYp
  GemmParams q = p;
  q.B0 = dyp;
  q.a_rows = nullptr;
  q.row_gate = nullptr;
  q.row_slot = nullptr;
  q.k_strip = 1;
  return launch_gemm_kernels(true, R_DOWN_WGRAD, q, max_m_tiles, s);
}

}  // namespace moe
