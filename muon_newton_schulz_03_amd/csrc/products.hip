// gfx950 (CDNA4) bf16 Newton-Schulz products of the Muon step.
//
// The iteration (overview page "The NanoGPT speedrun", paragraph "Six records
// account for most of the speedup", record #3: the update is driven towards
// its polar factor by Newton-Schulz steps):
//   stage 1  A = X X^T             (K = n)
//   stage 2  B = b A + c A A       (K = m; A is symmetric, so A A = A A^T)
//   stage 3  X <- a X + B X        (K = m); the last iteration applies the
//            weight step W <- W - lr scale O instead of storing X
//
// Design (one persistent kernel per product kind):
//   * the update's output tile is 256 rows x 128 columns per 256-thread block,
//     two blocks per CU; wave w owns rows 128 (w >> 1) .. +127 and columns
//     64 (w & 1) .. +63 as 4 x 2 v_mfma_f32_32x32x16_bf16 blocks (128
//     accumulator registers).  Per K step a wave reads 4 + 2 fragments from
//     LDS for 8 MFMAs, and a block moves 48 bytes from L2 per 512 FLOP-clocks
//     of its CU (64 for 128x128 tiles).  The polynomial takes the same tiles;
//     the Gram product takes 128 x 128 tiles (wave w: rows 64 (w >> 1),
//     columns 64 (w & 1), 2 x 2 blocks) for balance: its tiles' K (= n)
//     differs fourfold within a launch;
//   * X, its low bytes, A and B are stored in 128-row x 32-column tiles (each
//     tile contiguous), so a K slab of 32 elements of a 128-row panel is one
//     contiguous 8 KiB tile: every direct-to-LDS request reads 1 KiB of
//     contiguous memory (whole cache lines), and every 32 x 32 output block
//     is 2 KiB of contiguous memory;
//   * K streams in 32-element slabs through an LDS ring filled by
//     direct-to-LDS buffer loads (three 24 KiB slots for 256-row tiles, five
//     16 KiB slots for 128-row tiles); slab kt + slots - 1 is
//     requested as slab kt starts, and the ring runs on from one tile into the
//     next, so a tile's first slabs are in flight during the previous tile's
//     epilogue;
//   * A and B are stored in full.  Stages 1 and 2 compute only the tiles
//     that reach the upper triangle (at 128 granularity) and write every
//     element at (i, j) and at (j, i); diagonal 32-blocks are made exactly
//     symmetric first, and a tile on the diagonal reads its column panel from
//     the matching half of its row panel.  So every operand is read
//     K-contiguous (ds_read_b128), except X as the right operand of B X, read
//     with the transposing ds_read_b64_tr_b16;
//   * stage 3 adds a X inside the K loop: the X slab of K rows k0 .. k0 + 31
//     holds X at exactly the output rows k0 .. k0 + 31 of the tile's columns,
//     so the wave owning those rows reads them there (with X's low bytes,
//     copied into LDS beside the ring for those slabs) and adds a x to its
//     accumulators; the epilogue then only stores;
//   * the epilogue stages one 32 x 32 accumulator block at a time in LDS, per
//     wave and without block barriers, so that global accesses run along
//     rows; the inputs it still needs (A in stage 2, W in the weight step) are
//     requested blocks ahead, and the next tile's first waits allow for the
//     epilogue's stores still in flight.
#include "device_common.h"

namespace muon {
namespace {

constexpr int kTM = 256;                      // update tile rows (Q operand's panel); see Shape
constexpr int kTN = 128;                      // tile columns (P operand's panel)
constexpr int kBK = 32;                       // K elements per slab
constexpr int kHalf = 128 * 2 * kBK;          // one 128-row half slab: 8 KiB
constexpr int kSlot = 3 * kHalf;              // Q rows 0..127, Q rows 128..255, P
constexpr int kRing = 3;
constexpr int kLoBuf = kBK * kTN;             // X's low bytes of one slab: 4 KiB
constexpr int kLoBase = kRing * kSlot;        // two low-byte buffers after the ring
constexpr int kLds = kLoBase + 2 * kLoBuf;    // 80 KiB: two blocks per CU
constexpr int kBlock = 32 * 32 * 4;           // one staged 32 x 32 fp32 block per wave
constexpr int kBlocks = 2;                    // resident blocks per CU
constexpr uint32_t kOob = 0x80000000u;        // buffer offset past every resource: load 0, store dropped
constexpr int kDma = 6;                       // ring requests per wave per slab (stage 3)

// Tile shape per stage.  Stages 2 and 3 take 256 x 128 tiles: their K loop
// moves fewer L2-to-LDS bytes per FLOP than with 128-row tiles.  The Gram
// product (stage 1) takes 128 x 128 tiles: a tile's K is n, up to four times
// another's in one launch, and with 256-row tiles the launch waits for its
// longest tiles; its slots hold two 128-row panels, and the spare LDS buys a
// deeper ring.
template <int STAGE>
struct Shape {
  static constexpr bool kWide = STAGE != 1;
  static constexpr int kRows = kWide ? 256 : 128;   // tile rows
  static constexpr int kMI = kRows / 64;            // 32-row accumulator blocks per wave
  static constexpr int kSlot = kWide ? 3 * kHalf : 2 * kHalf;
  static constexpr int kPOff = kWide ? 2 * kHalf : kHalf;  // column panel inside a slot
  static constexpr int kRing = kWide ? 3 : 5;
  static constexpr int kAhead = kRing - 1;          // slabs requested ahead
  static constexpr int kDma = kSlot / 1024 / 4;     // requests per wave per slab
  static_assert(kWide || kRing * kSlot <= kLds, "ring fits the block's LDS");
  static_assert(4 * kBlock <= kSlot, "staged epilogue blocks fit one slot");
};

// Swizzles (16-byte chunk c of row r sits at chunk c ^ swz(r)).  Bank model,
// from rocprofv3 bank-conflict counts of each access pattern on gfx950:
// 16-byte reads serve 16 lanes per clock over 256 bytes, 8-byte reads 32
// lanes over 256 bytes, 4-byte reads 32 lanes over 128 bytes, and 16-byte
// writes 8 lanes over 128 bytes.
// K-contiguous half slab (64-byte rows): MFMA fragment reads (32 rows x one
// chunk per 32 lanes) conflict-free.
__device__ __forceinline__ int kc_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// X slab of B X (32 K rows x 128 columns, four 32-column tiles; in LDS as
// [tile][32 rows][64 bytes]): transposing fragment reads (4 K rows x 2 chunks
// per 16 lanes) conflict-free; the a X term's 8-byte row reads 2-way.
__device__ __forceinline__ int xs_swz(int k) { return (k >> 2) & 3; }
// Low bytes of that slab ([tile][32 rows][32 bytes], 16-byte halves of row k
// at half ^ lo_swz(k)): the a X term's 4-byte row reads 4-way.  Those two
// conflicts cost nothing measurable (16-byte reads without them: same step).
__device__ __forceinline__ int lo_swz(int k) { return (k >> 3) & 1; }
// Staged 32 x 32 fp32 block (128-byte rows): row-pass reads conflict-free,
// accumulator writes, row-pass writes and 4 x 4 block reads 2-way.  A
// swizzle that made the writes conflict-free, r ^ ((r >> 1) & 1), cost
// registers and no time.
__device__ __forceinline__ int st_swz(int r) { return (r >> 1) & 7; }

// Two of the eight 1 KiB instructions that fill a K-contiguous half slab
// from one contiguous 8 KiB tile (128 rows x 64 bytes): instruction n moves
// rows 16 n .. 16 n + 15, lane l row 16 n + l / 4 at physical chunk l % 4,
// i.e. logical chunk (l % 4) ^ kc_swz(row).
__device__ __forceinline__ void dma_half(char* lds, rsrc_t rs, uint32_t tile, int w, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int n = 2 * w + q;
    const int row = 16 * n + (lane >> 2);
    const uint32_t voff = tile + (uint32_t)row * 64u + 16u * (uint32_t)((lane & 3) ^ kc_swz(row));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MUON_LDS(lds + n * 1024), 16, voff, 0, 0, 0);
  }
}
// Two of the eight instructions that copy the X slab of B X: 32 K rows of
// four consecutive 32-column tiles, 2 KiB contiguous in each (`piece` is the
// first one's byte offset, the next ones follow 8 KiB apart); instruction n
// moves rows 16 (n % 2) .. +15 of tile n / 2.
__device__ __forceinline__ void dma_xslab(char* lds, rsrc_t rs, uint32_t piece, int w, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int n = 2 * w + q;
    const int k = 16 * (n & 1) + (lane >> 2);
    const uint32_t voff = piece + (uint32_t)(n >> 1) * 8192u + (uint32_t)k * 64u +
                          16u * (uint32_t)((lane & 3) ^ xs_swz(k));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MUON_LDS(lds + n * 1024), 16, voff, 0, 0, 0);
  }
}
// One of the four instructions that copy the X slab's low bytes (32 rows x 32
// bytes of four consecutive tiles, 1 KiB contiguous in each, 4 KiB apart):
// wave w moves tile w's rows.
__device__ __forceinline__ void dma_lo(char* lds, rsrc_t rs, uint32_t piece, int w, int lane) {
  const int k = lane >> 1;
  const uint32_t voff = piece + (uint32_t)w * 4096u + (uint32_t)k * 32u + 16u * (uint32_t)((lane & 1) ^ lo_swz(k));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MUON_LDS(lds + w * 1024), 16, voff, 0, 0, 0);
}

// Two transposing-read fragments of the X slab (columns base + 0..31 and
// base + 32..63, K step ks): in a 16-lane group, lane r addresses K row
// k0 + r / 4, columns J0 + 4 (r % 4) .. +3, and lane i receives K rows
// k0 .. k0 + 3 of column J0 + i, the MFMA operand layout.  The reads and their
// wait sit in one asm block: the compiler would otherwise wait for every
// in-flight direct-to-LDS load first.
__device__ __forceinline__ void frags_xs(u32x4 (&f)[2], const char* l, int base, int lane, int ks) {
  const int g = lane >> 4, r = lane & 15;
  uint32_t addr[2][2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int jel = base + n * 32 + 16 * (g & 1) + 4 * (r & 3);  // first of 4 columns
    const int tile = jel >> 5, chunk = (jel & 31) >> 3, half = (jel >> 2) & 1;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int k = 16 * ks + 8 * (g >> 1) + 4 * m + (r >> 2);
      addr[n][m] = (uint32_t)(uintptr_t)(l + tile * 2048 + k * 64 + ((chunk ^ xs_swz(k)) << 4) + (half << 3));
    }
  }
  u32x2 t00, t01, t10, t11;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t00), "=&v"(t01), "=&v"(t10), "=&v"(t11)
      : "v"(addr[0][0]), "v"(addr[0][1]), "v"(addr[1][0]), "v"(addr[1][1])
      : "memory");
  f[0] = u32x4{t00.x, t00.y, t01.x, t01.y};
  f[1] = u32x4{t10.x, t10.y, t11.x, t11.y};
}

// Where one tile's operands are (byte offsets into the tiled matrices).
struct Ctx {
  const void* q;            // row-panel source (X, A or B)
  const void* p;            // column-panel source (X or A); null: empty requests
  const uint8_t* xlo;       // stage 3 with the low bytes: X's low bytes
  uint32_t qbytes, pbytes;  // sizes of the two matrices
  uint32_t qoff;            // tile (row block of Q's rows 0..127, K slab 0)
  uint32_t qblk;            // bytes per 128-row block of Q's matrix
  uint32_t poff;            // stages 1, 2: tile (P's row block, K slab 0); stage 3: X tile (0, 4 tj)
  uint32_t pblk;            // bytes per 128-row block of P's matrix
  int nk;                   // K slabs
  int i0, j0;               // output origin
  int psrc;                 // 0: P from its own slab region; 1, 2: from Q half 0, 1 (on the diagonal)
  int skip1;                // 256-row tiles of stage 2: rows 128..255 lie below the diagonal
};

template <int STAGE, int MODE>
__device__ __forceinline__ Ctx ctx_of(const StageArgs& args, const Tile& tl) {
  const DevMat* m = args.mats + tl.mat;
  const uint32_t mp = (uint32_t)load_uniform(&m->mp), np = (uint32_t)load_uniform(&m->np);
  const void* xin = ((args.t - 1) & 1) ? load_uniform(&m->xo[1]) : load_uniform(&m->xo[0]);
  Ctx c;
  c.i0 = tl.ti * Shape<STAGE>::kRows;
  c.j0 = tl.tj * kTN;
  c.psrc = 0;
  c.skip1 = 0;
  c.xlo = nullptr;
  const uint32_t xb = mp * np * 2u, ab = mp * mp * 2u;
  if (STAGE == 1 || STAGE == 2) {
    const uint32_t K = STAGE == 1 ? np : mp;
    c.q = c.p = STAGE == 1 ? xin : (const void*)load_uniform(&m->a);
    c.qbytes = c.pbytes = STAGE == 1 ? xb : ab;
    c.qblk = c.pblk = K * 256u;  // (K / 32) tiles of 8 KiB
    c.qoff = (uint32_t)(c.i0 >> 7) * c.qblk;
    c.poff = (uint32_t)(c.j0 >> 7) * c.pblk;
    c.nk = (int)K / kBK;
    if (Shape<STAGE>::kWide) {  // the column panel is one of the row halves on the tile's diagonal
      const int rel = tl.tj - 2 * tl.ti;
      if (rel == 0 || rel == 1) c.psrc = rel + 1;
      c.skip1 = rel == 0;
    } else {
      c.psrc = tl.ti == tl.tj;
    }
  } else {
    c.q = load_uniform(&m->b);
    c.qbytes = ab;
    c.qblk = mp * 256u;
    c.qoff = (uint32_t)(c.i0 >> 7) * c.qblk;
    c.p = xin;
    c.pbytes = xb;
    c.pblk = np * 256u;
    c.poff = (uint32_t)(c.j0 >> 5) * 8192u;
    c.nk = (int)mp / kBK;
    if (MODE & kHiLo) c.xlo = load_uniform(&m->xlo);
  }
  return c;
}

// What B's stored diagonal lacks, per row i: the change of B_ii that the
// rounding of A_ii causes (the Gram epilogue stores it) plus B_ii - bf16(B_ii)
// (the polynomial epilogue adds it), as fp32 words right after B (4 mp bytes
// after its 2 mp mp).  Entry of row i: a lane's rows i0 + 32 mi + l % 32 (mi =
// 0..3) of a 128-row panel at i0 are four consecutive entries.
__device__ __forceinline__ uint32_t bres_entry(uint32_t i) {
  return 128u * (i >> 7) + 4u * (i & 31u) + ((i & 127u) >> 5);
}

// A tile's diagonal words for the rows a lane folds a*X into, rows R0 + 32 mi
// + lane % 32 (mi = 0..3) of the wave's 128-row panel at R0.  Update kernels
// that read X's low bytes hold them in registers: one 16-byte request per
// lane.  The others, short of registers in the weight step, keep the panel's
// 512 bytes in the unused low-byte buffers instead, copied by two 4-byte
// direct-to-LDS requests per lane, and read a lane's word at each fold.  Either request moves nothing for an empty tile,
// which still issues it so that the wait counts stay static.
__device__ __forceinline__ rsrc_t res_rsrc(const Ctx& c) {
  return make_rsrc(c.q, c.p ? c.qbytes + (c.qblk >> 6) : 0u);  // stage 3: c.q is B (c.qbytes = 2 mp mp), 4 mp = c.qblk / 64
}
__device__ __forceinline__ u32x4 issue_res_regs(const Ctx& c, int R0, int lane) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       res_rsrc(c), c.qbytes + 4u * bres_entry((uint32_t)R0 + (uint32_t)(lane & 31)), 0, 0));
}
__device__ __forceinline__ void issue_res_lds(char* dst, const Ctx& c, int R0, int lane) {
  const rsrc_t rs = res_rsrc(c);
  const uint32_t off = c.qbytes + 512u * (uint32_t)(R0 >> 7) + 4u * (uint32_t)lane;
#pragma unroll
  for (int h = 0; h < 2; ++h) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MUON_LDS(dst + 256 * h), 4, off + 256u * h, 0, 0, 0);
}
// The LDS copy: half `half` (tiles take the two low-byte buffers in turn, so
// that the next tile's words can land while this tile's are read), 1 KiB per
// wave; lane l's word of block mi at + 16 (l % 32) + 4 mi.
__device__ __forceinline__ char* res_lds(char* smem, int half, int w) { return smem + kLoBase + kLoBuf * half + 1024 * w; }
__device__ __forceinline__ float read_res(const char* src, int lane, int mi) {
  return *(const float*)(src + 16 * (lane & 31) + 4 * mi);
}
// Word of block mi (0..3) of those rows.
__device__ __forceinline__ float res_of(u32x4 r, int mi) {
  const uint32_t lo = mi & 1 ? r.y : r.x, hi = mi & 1 ? r.w : r.z;
  return __uint_as_float(mi < 2 ? lo : hi);
}

// Request slab kt of a tile into ring slot `slot` (kDma instructions per wave;
// parts the tile does not need get empty resources, which move nothing).
template <int STAGE>
__device__ __forceinline__ void issue_slab(char* smem, const Ctx& c, int kt, int slot, int w, int lane) {
  using G = Shape<STAGE>;
  char* s = smem + slot * G::kSlot;
  const uint32_t kb = (uint32_t)kt * 8192u;
  dma_half(s, make_rsrc(c.q, c.p ? c.qbytes : 0u), c.qoff + kb, w, lane);
  if (G::kWide) dma_half(s + kHalf, make_rsrc(c.q, c.p && !c.skip1 ? c.qbytes : 0u), c.qoff + c.qblk + kb, w, lane);
  const rsrc_t p = make_rsrc(c.p, c.p && !c.psrc ? c.pbytes : 0u);
  if (STAGE == 3)
    dma_xslab(s + G::kPOff, p, c.poff + (uint32_t)(kt >> 2) * c.pblk + (uint32_t)(kt & 3) * 2048u, w, lane);
  else
    dma_half(s + G::kPOff, p, c.poff + kb, w, lane);
}

// Request X's low bytes of slab kt into low-byte buffer `buf` (1 instruction
// per wave; empty unless the slab's K rows are output rows of the tile).
__device__ __forceinline__ void issue_lo(char* smem, const Ctx& c, int kt, int buf, int w, int lane) {
  const bool need = c.p && kt * kBK >= c.i0 && kt * kBK < c.i0 + kTM;  // stage 3 only
  dma_lo(smem + kLoBase + buf * kLoBuf, make_rsrc(c.xlo, need ? (c.pbytes >> 1) : 0u),
         (c.poff >> 1) + (uint32_t)(kt >> 2) * (c.pblk >> 1) + (uint32_t)(kt & 3) * 1024u, w, lane);
}

// Per-lane byte offsets of the K-contiguous fragment reads: lane l reads row
// 32 m + l % 32 of a half at logical chunk 2 ks + l / 32.
struct FragOff {
  uint32_t row, ch[2];
};
__device__ __forceinline__ FragOff frag_off(int lane) {
  FragOff f;
  const int r = lane & 31, sw = kc_swz(r);
  f.row = (uint32_t)r * 64u;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) f.ch[ks] = (uint32_t)(((2 * ks + (lane >> 5)) ^ sw) << 4);
  return f;
}

// One slab: acc[mi][nj] += P(columns) x Q(rows)^T over 32 K.  MFMA operand A
// is the P fragment (MFMA row <-> output column), operand B the Q fragment,
// so lane l holds output row 32 mi + l % 32 and 4 consecutive output columns
// per group of 4 accumulator registers.
template <bool PX, int MI>
__device__ __forceinline__ void mma_slab(f32x16 (&acc)[MI][2], const char* qh, const char* p, int wn, int lane,
                                         const FragOff& fo) {
  u32x4 qf[2][MI], pf[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) qf[ks][mi] = *(const u32x4*)(qh + mi * 2048 + fo.row + fo.ch[ks]);
    if (PX) {
      frags_xs(pf[ks], p, 64 * wn, lane, ks);
    } else {
#pragma unroll
      for (int nj = 0; nj < 2; ++nj) pf[ks][nj] = *(const u32x4*)(p + (2 * wn + nj) * 2048 + fo.row + fo.ch[ks]);
    }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nj = 0; nj < 2; ++nj)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pf[ks][nj]),
                                                               __builtin_bit_cast(bf16x8, qf[ks][mi]), acc[mi][nj],
                                                               0, 0, 0);
}

// Stage 3: acc block row mi += alpha x, x = X at the output rows that the X
// slab in LDS holds (K row l % 32 of the slab is output row 32 mi + l % 32 of
// the wave), decoded with its low bytes when LO.
template <bool LO>
__device__ __forceinline__ void fold_x(f32x16 (&a)[2], const char* p, const char* lo, int wn, int lane, float alpha) {
  const int k = lane & 31, h = lane >> 5;
#pragma unroll
  for (int nj = 0; nj < 2; ++nj)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tile = 2 * wn + nj;  // the 32-column tile of these 4 columns
      const u32x2 hi = *(const u32x2*)(p + tile * 2048 + k * 64 + ((g ^ xs_swz(k)) << 4) + 8 * h);
      float x[4];
      if (LO) {
        const uint32_t lw =
            *(const uint32_t*)(lo + tile * 1024 + k * 32 + (((g >> 1) ^ lo_swz(k)) << 4) + 8 * (g & 1) + 4 * h);
        unpack4_hilo(hi, lw, x);
      } else {
        unpack4_bf16(hi, x);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) a[nj][4 * g + e] = fmaf(alpha, x[e], a[nj][4 * g + e]);
    }
}

// ------------------------------------------------------------- epilogue --

// The wave's staged 32 x 32 fp32 block (128-byte rows).
struct Stage {
  char* base;
  __device__ __forceinline__ f32x4* at(int r, int cc) const {
    return (f32x4*)(base + r * 128 + ((cc ^ st_swz(r)) << 4));
  }
  __device__ __forceinline__ float* elem(int r, int col) const {
    return (float*)(base + r * 128 + (((col >> 2) ^ st_swz(r)) << 4)) + (col & 3);
  }
  // accumulator block: lane l holds row l % 32, columns 8 g + 4 (l / 32) .. +3
  __device__ __forceinline__ void put(const f32x16& a, int lane) const {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int g = 0; g < 4; ++g) *at(r, 2 * g + h) = f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
  }
};

// Row pass p (0, 1): lane l handles row 16 p + l / 4, columns 8 (l % 4) .. +7.
__device__ __forceinline__ int rp_row(int p, int lane) { return 16 * p + (lane >> 2); }
__device__ __forceinline__ int rp_col(int lane) { return 8 * (lane & 3); }
// Block pass: lane l handles the 4 x 4 block at rows 4 (l % 8) .., columns 4 (l / 8) ..
__device__ __forceinline__ int bp_row(int lane) { return 4 * (lane & 7); }
__device__ __forceinline__ int bp_col(int lane) { return 4 * (lane >> 3); }

__device__ __forceinline__ void read8(const Stage& st, int r, int c, float* v) {
  const f32x4 x = *st.at(r, c >> 2), y = *st.at(r, (c >> 2) + 1);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
}
__device__ __forceinline__ void write8(const Stage& st, int r, int c, const float* v) {
  *st.at(r, c >> 2) = f32x4{v[0], v[1], v[2], v[3]};
  *st.at(r, (c >> 2) + 1) = f32x4{v[4], v[5], v[6], v[7]};
}
// blk[e][f] = block[r + e][c + f]
__device__ __forceinline__ void read_block(const Stage& st, int r, int c, float (&blk)[4][4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4 x = *st.at(r + e, c >> 2);
    blk[e][0] = x.x; blk[e][1] = x.y; blk[e][2] = x.z; blk[e][3] = x.w;
  }
}
// A diagonal 32-block of A or B: strictly lower elements take the values of
// their mirrors, so that the block is exactly symmetric (reads before writes).
__device__ __forceinline__ void symmetrize(const Stage& st, int lane) {
  const int r = lane & 31, c0 = 16 * (lane >> 5);
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = c0 + e < r ? *st.elem(c0 + e, r) : 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if (c0 + e < r) *st.elem(r, c0 + e) = v[e];
}

__device__ __forceinline__ void store_b128(rsrc_t rs, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), rs,
                                         off, 0, 0);
}
__device__ __forceinline__ void store_b64(rsrc_t rs, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), rs,
                                        off, 0, 0);
}

// Weight step (stage 3, last iteration), W element (R, C) of the caller's
// row-major matrix.  The common case, fp32 W with rows of a multiple of 4
// elements on 16-byte boundaries ("fast"), takes 16-byte accesses requested
// blocks ahead, all issued (out-of-range lanes get an offset past the
// resource) so that the instruction counts are static; any other W (bf16,
// ragged rows) takes a compact element-by-element loop.
struct WRes {
  rsrc_t r;
  int rows, cols, bf16, fast;
  float lr;
};
__device__ __forceinline__ uint32_t woff(const WRes& w, int R, int C) {
  return R < w.rows && C < w.cols ? ((uint32_t)R * (uint32_t)w.cols + (uint32_t)C) << 2 : kOob;
}
__device__ __forceinline__ u32x4 wload4(const WRes& w, int R, int C) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.r, woff(w, R, C), 0, 0));
}
__device__ __forceinline__ void wstore4(const WRes& w, int R, int C, const float* v) {
  store_b128(w.r, woff(w, R, C),
             u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
}
// W (R, C) -= lr * o for one element of any W (bounds-checked, not unrolled)
__device__ __forceinline__ void wstep1(const WRes& w, int R, int C, float o) {
  if (R >= w.rows || C >= w.cols) return;
  const uint32_t e = (uint32_t)R * (uint32_t)w.cols + (uint32_t)C;
  if (w.bf16) {
    const float x = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(w.r, e << 1, 0, 0) << 16);
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f2bf(fmaf(-w.lr, o, x)), w.r, e << 1, 0, 0);
  } else {
    const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(w.r, e << 2, 0, 0));
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(-w.lr, o, x)), w.r, e << 2, 0, 0);
  }
}

// vmcnt(n), rounded down to the nearest supported immediate (waiting for more
// than needed is always correct); n is wave-uniform.
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 62) MUON_WAIT_VMCNT(62);
  else if (n >= 56) MUON_WAIT_VMCNT(56);
  else if (n >= 48) MUON_WAIT_VMCNT(48);
  else if (n >= 40) MUON_WAIT_VMCNT(40);
  else if (n >= 32) MUON_WAIT_VMCNT(32);
  else if (n >= 28) MUON_WAIT_VMCNT(28);
  else if (n >= 24) MUON_WAIT_VMCNT(24);
  else if (n >= 20) MUON_WAIT_VMCNT(20);
  else if (n >= 16) MUON_WAIT_VMCNT(16);
  else if (n >= 12) MUON_WAIT_VMCNT(12);
  else if (n >= 8) MUON_WAIT_VMCNT(8);
  else if (n >= 6) MUON_WAIT_VMCNT(6);
  else if (n >= 4) MUON_WAIT_VMCNT(4);
  else MUON_WAIT_VMCNT(0);
}

// Epilogue of one wave over its 32 x 32 accumulator blocks (b = 2 mi + nj:
// eight in stage 3, four in stages 1 and 2).  Inputs per block (A of stage 2 at the direct positions, W of the
// weight step) are requested kDepth blocks ahead.
template <int STAGE, int MODE>
struct Epi {
  static constexpr bool kUpd = STAGE == 3;
  static constexpr bool kLastIt = kUpd && (MODE & kLast);
  static constexpr bool kLoOut = kUpd && !kLastIt && (MODE & kWriteLo);
  static constexpr int kDepth = STAGE == 2 ? 3 : (kLastIt ? 2 : 0);
  static constexpr int kInSlots = kDepth > 0 ? kDepth : 1;
  static constexpr int kMI = Shape<STAGE>::kMI;
  static constexpr int kNB = 2 * kMI;  // the wave's 32 x 32 blocks
  struct In {
    u32x4 v[4];  // stage 2: A of row passes 0, 1 (bf16); weight step: W as fp32 bit patterns
  };

  int R0, C0;    // the wave's canonical origin
  int lane, t;
  float cb, cc, pre;
  float dbs;     // stage 1: the factor of the polynomial's b and c (s at t = 1, else 1)
  void* bmat;    // stage 1: B, whose diagonal words the Gram epilogue stores
  void* out;     // stage 1: A; stage 2: B; stage 3: the new X
  uint32_t resoff;  // stages 1, 2: this lane's diagonal word for a diagonal block at rows R0.. (byte offset
                    // from B; kOob for lanes >= 32)
  uint8_t* xlo;
  const void* ain;
  uint32_t mp, np;
  int transposed;
  WRes w;
  int sub, tj;   // 128-row subtile of the wave's rows; 128-column tile

  __device__ __forceinline__ Epi(const StageArgs& args, const DevMat* m, const Ctx& c, int wm, int wn, int lane_)
      : lane(lane_) {
    R0 = c.i0 + (Shape<STAGE>::kRows / 2) * wm;
    C0 = c.j0 + 64 * wn;
    sub = R0 >> 7;
    tj = c.j0 >> 7;
    t = args.t;
    cb = args.b;
    cc = args.c;
    pre = 1.f;
    dbs = 1.f;
    if (args.t == 1 && STAGE != 3) {  // the first iteration works on U = X0 / s (s = 1 / (||U|| + eps))
      const float s = load_uniform(load_uniform(&m->sc));
      if (STAGE == 1) pre = s * s, dbs = s;
      if (STAGE == 2) cb *= s, cc *= s;
    }
    mp = (uint32_t)load_uniform(&m->mp);
    np = (uint32_t)load_uniform(&m->np);
    resoff = lane < 32 ? mp * mp * 2u + 4u * bres_entry((uint32_t)(R0 + lane)) : kOob;
    bmat = STAGE == 1 ? load_uniform(&m->b) : nullptr;
    xlo = nullptr;
    ain = nullptr;
    out = nullptr;
    transposed = 0;
    if (STAGE == 1) out = load_uniform(&m->a);
    if (STAGE == 2) out = load_uniform(&m->b), ain = c.q;
    if (STAGE == 3 && !kLastIt) {
      out = (args.t & 1) ? load_uniform(&m->xo[1]) : load_uniform(&m->xo[0]);
      if (kLoOut) xlo = load_uniform(&m->xlo);
    }
    if (kLastIt) {
      transposed = load_uniform(&m->transposed);
      w.bf16 = load_uniform(&m->w_bf16);
      w.rows = load_uniform(&m->rows);
      w.cols = load_uniform(&m->cols);
      w.fast = !w.bf16 && load_uniform(&m->vec_w);
      w.lr = args.lr * load_uniform(&m->scale);
      w.r = make_rsrc(load_uniform(&m->w), (uint32_t)w.rows * (uint32_t)w.cols * (w.bf16 ? 2u : 4u));
    }
  }

  __device__ __forceinline__ int br(int b) const { return R0 + 32 * (b >> 1); }
  __device__ __forceinline__ int bc(int b) const { return C0 + 32 * (b & 1); }

  // block kinds of the symmetric products
  enum { kOff = 0, kDiag = 1, kLower = 2 };
  __device__ __forceinline__ int kind(int b) const {
    if (sub < tj) return kOff;
    const int dr = (R0 & 127) + 32 * (b >> 1), dc = (C0 & 127) + 32 * (b & 1);  // offsets in the diagonal subtile
    return dr < dc ? kOff : dr == dc ? kDiag : kLower;
  }

  // vector-memory instructions of one block's input requests and of its stores
  __device__ __forceinline__ int loads_per_block() const {
    if (STAGE == 2) return 2;
    if (kLastIt) return w.fast ? 4 : 0;
    return 0;
  }
  __device__ __forceinline__ int stores_per_block() const {
    if (STAGE != 3) return 6;  // stage 2 issues one more (see process): counted as 6, waits only get stricter
    if (!kLastIt) return kLoOut ? 4 : 2;
    return w.fast ? 4 : 0;
  }

  __device__ __forceinline__ void load(int b, In& in) const {
    if (STAGE == 2) {
      const uint32_t t0 = tiled(br(b), bc(b), mp);  // the block: 2 KiB contiguous
#pragma unroll
      for (int p = 0; p < 2; ++p)
        in.v[p] = *gv<u32x4>((const uint16_t*)ain + t0 + rp_row(p, lane) * 32 + rp_col(lane));
    }
    if (kLastIt && w.fast) {
      if (!transposed) {  // W row = canonical row: row pass p, halves h
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            in.v[2 * p + h] = wload4(w, br(b) + rp_row(p, lane), bc(b) + rp_col(lane) + 4 * h);
      } else {  // W row = canonical column: block pass, f = 0..3
#pragma unroll
        for (int f = 0; f < 4; ++f) in.v[f] = wload4(w, bc(b) + bp_col(lane) + f, br(b) + bp_row(lane));
      }
    }
  }

  __device__ __forceinline__ void process(int b, const Stage& st, const In& in) const {
    const int r0 = br(b), c0 = bc(b);
    if (kUpd) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int r = rp_row(p, lane), c = rp_col(lane);
        float v[8];
        read8(st, r, c, v);
        if (!kLastIt) {
          const uint32_t off = tiled(r0, c0, np) + r * 32 + c;  // the block: 2 KiB contiguous
          const u32x4 hi = pack8_bf16(v);
          __builtin_nontemporal_store(hi, gv<u32x4>((uint16_t*)out + off));
          if (kLoOut) __builtin_nontemporal_store(lo8(v, hi), gv<u32x2>(xlo + off));
        } else if (w.fast && !transposed) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float wv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[e] = fmaf(-w.lr, v[4 * h + e], __uint_as_float(in.v[2 * p + h][e]));
            wstore4(w, r0 + r, c0 + c + 4 * h, wv);
          }
        }
      }
      if (kLastIt && !w.fast) {  // any other W: element by element, lanes along W's rows
#pragma unroll 1
        for (int q = 0; q < 16; ++q) {
          const int i = lane + 64 * q, a = i >> 5, b2 = i & 31;
          const int r = transposed ? b2 : a, c = transposed ? a : b2;
          const float o = *st.elem(r, c);
          if (transposed)
            wstep1(w, c0 + c, r0 + r, o);
          else
            wstep1(w, r0 + r, c0 + c, o);
        }
      }
      if (kLastIt && w.fast && transposed) {
        float blk[4][4];
        read_block(st, bp_row(lane), bp_col(lane), blk);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          float wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) wv[e] = fmaf(-w.lr, blk[e][f], __uint_as_float(in.v[f][e]));
          wstore4(w, c0 + bp_col(lane) + f, r0 + bp_row(lane), wv);
        }
      }
      return;
    }
    // stages 1 and 2: A or B, written at (i, j) and at (j, i)
    const int k = kind(b);
    if (k == kDiag) symmetrize(st, lane);
    const rsrc_t o_rs = make_rsrc(out, mp * mp * 2u);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = rp_row(p, lane), c = rp_col(lane);
      float v[8];
      read8(st, r, c, v);
      if (STAGE == 1) {
        if (t == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= pre;
        }
      } else {
        float av[8];
        unpack8_bf16(in.v[p], av);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(cc, v[e], cb * av[e]);
      }
      const uint32_t o = k != kLower ? (tiled(r0, c0, mp) + r * 32 + c) * 2u : kOob;
      store_b128(o_rs, o, pack8_bf16(v));
      if (STAGE == 2 || t == 1) write8(st, r, c, v);  // the mirrored writes take the final values
    }
    {
      // The diagonal went out as bf16 like every element.  The staged block
      // now holds the final values: lane l < 32 takes element (l, l) of a
      // diagonal block (row R0 + 32 (b / 2) + l: entry bres_entry(R0 + l) +
      // b / 2), and r = x - bf16(x) is what the rounding left out.  Into B's
      // diagonal word of that row:
      //   stage 1 stores the change of B_ii that r causes, (b + 2 c A_ii) r,
      //     with the polynomial's b and c (both times s at t = 1);
      //   stage 2 adds r (an atomic add, which returns nothing to wait for).
      // Every block issues the request (out of range elsewhere), and it is
      // left out of the instruction counts the waits use: an uncounted
      // request in flight only makes a wait stricter.
      const float x = *st.elem(lane & 31, lane & 31);
      const float r = x - bf2f(f2bf(x));
      const uint32_t doff = k == kDiag ? resoff + 4u * (uint32_t)(b >> 1) : kOob;
      const rsrc_t w_rs = make_rsrc(STAGE == 1 ? bmat : out, mp * mp * 2u + mp * 4u);
      if (STAGE == 1)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dbs * fmaf(2.f * cc, x, cb) * r), w_rs, doff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(r, w_rs, doff, 0, 0);
    }
    float blk[4][4];
    const int r = bp_row(lane), c = bp_col(lane);
    read_block(st, r, c, blk);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t o = k == kOff ? (tiled(c0, r0, mp) + (c + f) * 32 + r) * 2u : kOob;
      store_b64(o_rs, o, pack4_bf16(blk[0][f], blk[1][f], blk[2][f], blk[3][f]));
    }
  }

  // The whole epilogue.  `vm_pre`: vector-memory instructions issued after
  // the requests of blocks 0 .. kDepth - 1 (made during the tile's last
  // slabs).  Block b + kDepth's inputs are requested once block b has been
  // processed (its input registers are then free).  Returns the instructions
  // the epilogue itself issued.
  __device__ __forceinline__ int run(const f32x16 (&acc)[kMI][2], const Stage& st, In (&in)[kInSlots],
                                     int vm_pre) const {
    const int lpb = loads_per_block(), spb = stores_per_block();
    int issued = 0;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      st.put(acc[b >> 1][b & 1], lane);
      if (kDepth > 0 && lpb > 0) {
        // instructions issued after block b's request, which may stay in flight
        int after;
        if (b < kDepth) {
          after = (kDepth - 1 - b) * lpb + vm_pre + issued;
        } else {
          const int last_req = b + kDepth - 1 < kNB ? b + kDepth - 1 : kNB - 1;
          after = (kDepth - 1) * spb + (last_req - b) * lpb;
        }
        wait_vm(after);
      }
      process(b, st, in[b % kInSlots]);
      issued += spb;
      if (kDepth > 0 && lpb > 0 && b + kDepth < kNB) {
        load(b + kDepth, in[(b + kDepth) % kInSlots]);
        issued += lpb;
      }
    }
    return issued;
  }
};

// Requests of a tile's first slabs (and of its first low bytes) into ring
// slots 0 .. kAhead - 1 and low-byte buffer 0: the start of a block's run of
// tiles, with nothing of the ring in flight.  Stage 3 first requests the
// tile's diagonal words of B (returned when held in registers; in LDS half 0
// otherwise).
template <int STAGE, int MODE>
__device__ __forceinline__ u32x4 tile_prologue(char* smem, const Ctx& c, int w, int wm, int lane) {
  u32x4 res = {0u, 0u, 0u, 0u};
  if (STAGE == 3 && (MODE & kHiLo)) res = issue_res_regs(c, c.i0 + 128 * wm, lane);
  if (STAGE == 3 && !(MODE & kHiLo)) issue_res_lds(res_lds(smem, 0, w), c, c.i0 + 128 * wm, lane);
  if (STAGE == 3 && (MODE & kHiLo)) issue_lo(smem, c, 0, 0, w, lane);
#pragma unroll
  for (int d = 0; d < Shape<STAGE>::kAhead; ++d) issue_slab<STAGE>(smem, c, d, d, w, lane);
  // the register copy has landed once those are requested (the compiler sees
  // the wait and adds none of its own where the words are used)
  if (STAGE == 3 && (MODE & kHiLo)) MUON_WAIT_VMCNT(Shape<STAGE>::kAhead * Shape<STAGE>::kDma);
  return res;
}

// One tile: its K loop, whose last slabs request the first slabs of the
// block's next tile `cn` (cn.p == nullptr: empty requests, which keep the
// wait counts static), and its epilogue.  `g` counts the slabs the block has
// consumed (ring slot g % kRing, low-byte buffer g % 2); `pend` is the number
// of the previous epilogue's instructions issued after this tile's first
// kAhead slabs.  Stage 3: `res` and LDS half `half` hold the tile's diagonal
// words of B; the next tile's are requested into `resn` or the other
// half, just before its second slab.  Returns the instructions this tile's
// epilogue issued after the next tile's first slabs.
template <int STAGE, int MODE>
__device__ __forceinline__ int tile_pass(const StageArgs& args, char* smem, const Tile& tl, const Ctx& c,
                                         const Ctx& cn, int& g, int pend, int w, int wm, int wn, int lane,
                                         const FragOff& fo, u32x4 res, u32x4& resn, int half) {
  using E = Epi<STAGE, MODE>;
  using G = Shape<STAGE>;
  constexpr bool kLoIn = STAGE == 3 && (MODE & kHiLo);
  constexpr int kDepth = E::kDepth;
  constexpr int kAhead = G::kAhead;
  constexpr int kD = G::kDma;  // requests per wave per slab
  // on a diagonal tile of stages 1 and 2, waves whose rows lie wholly below
  // the diagonal only move data
  const bool idle = STAGE != 3 && (G::kWide ? wm == 1 && c.skip1 : c.psrc && wm == 1 && wn == 0);
  const int R0 = c.i0 + (G::kRows / 2) * wm;
  float alpha = args.a;
  if (STAGE == 3 && args.t == 1) alpha *= load_uniform(load_uniform(&args.mats[tl.mat].sc));
  typename E::In in[E::kInSlots];

  f32x16 acc[G::kMI][2];
#pragma unroll
  for (int mi = 0; mi < G::kMI; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][nj][v] = 0.f;

  // K slabs: at least kAhead (Gram: K = np >= 128, four slabs); stage 2 has
  // K = mp >= 256, so its first and last kAhead slabs never overlap
  const int nk = c.nk;
  // stage 2: the epilogue's first A requests, made as slab nk - kAhead starts
  const int early = STAGE == 2 && !idle ? kDepth * 2 : 0;
  int vm_pre = 0;  // instructions issued after those requests
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's part of slab kt (and its low bytes) has landed: only the
    // slabs requested after it may still be in flight, plus, at the first
    // slabs of a tile, the previous epilogue's instructions, and at the last
    // slabs of stage 2, the early A requests
    if (STAGE == 3) {
      if (kt == 0 || (kt == 1 && !kLoIn))
        wait_vm(kD + pend);
      else
        MUON_WAIT_VMCNT(kD);
    } else if (kt < kAhead) {
      wait_vm((kAhead - 1) * kD + pend);
    } else if (STAGE == 2 && kt > nk - kAhead) {
      wait_vm((kAhead - 1) * kD + early);
    } else {
      MUON_WAIT_VMCNT((kAhead - 1) * kD);
    }
    MUON_LDS_BARRIER();  // every wave's part has landed; slab kt - 1's slot is free
    if (kLoIn) issue_lo(smem, kt + 1 < nk ? c : cn, kt + 1 < nk ? kt + 1 : kt + 1 - nk, (g + 1) & 1, w, lane);
    if (STAGE == 2 && kt == nk - kAhead && !idle) {  // the epilogue's first inputs
      const E ep(args, args.mats + tl.mat, c, wm, wn, lane);
#pragma unroll
      for (int b = 0; b < kDepth; ++b) ep.load(b, in[b % E::kInSlots]);
    }
    if (STAGE == 3 && kt == nk - 1) {  // the next tile's diagonal words, before its second slab
      if (kLoIn)
        resn = issue_res_regs(cn, cn.i0 + 128 * wm, lane);
      else
        issue_res_lds(res_lds(smem, half ^ 1, w), cn, cn.i0 + 128 * wm, lane);
    }
    const int slot = (g + kAhead) % G::kRing;
    if (kt + kAhead < nk)
      issue_slab<STAGE>(smem, c, kt + kAhead, slot, w, lane);
    else
      issue_slab<STAGE>(smem, cn, kt + kAhead - nk, slot, w, lane);
    if (STAGE == 2 && kt >= nk - kAhead) vm_pre += kD;
    const char* s = smem + (g % G::kRing) * G::kSlot;
    if (!idle) {
      const char* p = c.psrc ? s + (c.psrc - 1) * kHalf : s + G::kPOff;
      if (STAGE == 3) {
        const int rel = kt * kBK - R0;  // this slab's K rows are output rows of the wave
        if (rel >= 0 && rel < 128) {
          const char* lo = smem + kLoBase + (g & 1) * kLoBuf;
          const float al = alpha + (kLoIn ? res_of(res, rel >> 5) : read_res(res_lds(smem, half, w), lane, rel >> 5));
          switch (rel >> 5) {
            case 0: fold_x<kLoIn>(acc[0], p, lo, wn, lane, al); break;
            case 1: fold_x<kLoIn>(acc[1], p, lo, wn, lane, al); break;
            case 2: fold_x<kLoIn>(acc[2 % G::kMI], p, lo, wn, lane, al); break;
            default: fold_x<kLoIn>(acc[3 % G::kMI], p, lo, wn, lane, al); break;
          }
        }
        mma_slab<true, G::kMI>(acc, s + wm * kHalf, p, wn, lane, fo);
      } else {
        mma_slab<false, G::kMI>(acc, s + wm * (G::kWide ? kHalf : kHalf / 2), p, wn, lane, fo);
      }
    }
    ++g;
  }

  // epilogue: the last slab's slot holds the waves' staged blocks
  MUON_LDS_BARRIER();  // all waves are done with the last slab
  int issued = 0;
  if (!idle) {
    const E ep(args, args.mats + tl.mat, c, wm, wn, lane);
    int early_w = 0;  // requests made after the next tile's first slabs, before run()
    if (E::kLastIt) {  // the weight step requests its first W blocks here (registers are short in the loop)
#pragma unroll
      for (int b = 0; b < kDepth; ++b) ep.load(b, in[b % E::kInSlots]);
      vm_pre = 0;
      early_w = kDepth * ep.loads_per_block();
    }
    Stage st;
    st.base = smem + ((g + G::kRing - 1) % G::kRing) * G::kSlot + w * kBlock;
    issued = early_w + ep.run(acc, st, in, vm_pre);
  }
  return issued;
}

// Persistent product kernel: block b takes the table entries b, b + G,
// b + 2 G, ... (G = gridDim.x, a multiple of 8: every entry stays on the XCD
// the table placed it on).
template <int STAGE, int MODE>
__global__ __launch_bounds__(kThreads, kBlocks) void ns_bf16_kernel(StageArgs args) {
  using E = Epi<STAGE, MODE>;
  using G = Shape<STAGE>;
  constexpr bool kLoIn = STAGE == 3 && (MODE & kHiLo);
  constexpr int kDepth = E::kDepth;
  constexpr int kAhead = G::kAhead;
  constexpr int kD = G::kDma;  // requests per wave per slab
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x;
  const FragOff fo = frag_off(lane);

  uint64_t raw = 0;
  int q = next_entry(args, blockIdx.x, stride, raw);
  if (q >= args.ntiles) return;
  Tile tl = tile_of(raw);
  Ctx c = ctx_of<STAGE, MODE>(args, tl);
  // stage 3: B's diagonal words (what its stored diagonal lacks) for the rows
  // this lane folds a*X into (issue_res_regs, issue_res_lds): the first
  // tile's requested here, each next tile's just before its second slab, so
  // that the wait for its first slab covers them.  res, resn: this tile's and
  // the next one's when held in registers; LDS half `half` otherwise.
  u32x4 res = {0u, 0u, 0u, 0u}, resn = res;
  int half = 0;
  if (STAGE == 3 && kLoIn) res = issue_res_regs(c, c.i0 + 128 * wm, lane);
  if (STAGE == 3 && !kLoIn) issue_res_lds(res_lds(smem, 0, w), c, c.i0 + 128 * wm, lane);
  if (kLoIn) issue_lo(smem, c, 0, 0, w, lane);
#pragma unroll
  for (int d = 0; d < kAhead; ++d) issue_slab<STAGE>(smem, c, d, d, w, lane);
  // the register copy has landed once those are requested (the compiler sees
  // the wait and adds none of its own where the words are used)
  if (STAGE == 3 && kLoIn) MUON_WAIT_VMCNT(kAhead * kD);
  int g = 0;     // slabs consumed by this block so far (ring slot g % kRing, low-byte buffer g % 2)
  int pend = 0;  // the previous epilogue's instructions, issued after this tile's first kAhead slabs
  for (;;) {
    // the block's next tile, for the requests that run ahead into it
    uint64_t rawn = 0;
    const int qn = next_entry(args, q + stride, stride, rawn);
    const bool more = qn < args.ntiles;
    const Tile tn = tile_of(rawn);
    Ctx cn = c;
    if (more)
      cn = ctx_of<STAGE, MODE>(args, tn);
    else
      cn.p = nullptr;  // empty requests keep the wait counts static
    // on a diagonal tile of stages 1 and 2, waves whose rows lie wholly below
    // the diagonal only move data
    const bool idle = STAGE != 3 && (G::kWide ? wm == 1 && c.skip1 : c.psrc && wm == 1 && wn == 0);
    const int R0 = c.i0 + (G::kRows / 2) * wm;
    float alpha = args.a;
    if (STAGE == 3 && args.t == 1) alpha *= load_uniform(load_uniform(&args.mats[tl.mat].sc));
    typename E::In in[E::kInSlots];

    f32x16 acc[G::kMI][2];
#pragma unroll
    for (int mi = 0; mi < G::kMI; ++mi)
#pragma unroll
      for (int nj = 0; nj < 2; ++nj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mi][nj][v] = 0.f;

    // K slabs: at least kAhead (Gram: K = np >= 128, four slabs); stage 2 has
    // K = mp >= 256, so its first and last kAhead slabs never overlap
    const int nk = c.nk;
    // stage 2: the epilogue's first A requests, made as slab nk - kAhead starts
    const int early = STAGE == 2 && !idle ? kDepth * 2 : 0;
    int vm_pre = 0;  // instructions issued after those requests
    for (int kt = 0; kt < nk; ++kt) {
      // this wave's part of slab kt (and its low bytes) has landed: only the
      // slabs requested after it may still be in flight, plus, at the first
      // slabs of a tile, the previous epilogue's instructions, and at the last
      // slabs of stage 2, the early A requests
      if (STAGE == 3) {
        if (kt == 0 || (kt == 1 && !kLoIn))
          wait_vm(kD + pend);
        else
          MUON_WAIT_VMCNT(kD);
      } else if (kt < kAhead) {
        wait_vm((kAhead - 1) * kD + pend);
      } else if (STAGE == 2 && kt > nk - kAhead) {
        wait_vm((kAhead - 1) * kD + early);
      } else {
        MUON_WAIT_VMCNT((kAhead - 1) * kD);
      }
      MUON_LDS_BARRIER();  // every wave's part has landed; slab kt - 1's slot is free
      if (kLoIn) issue_lo(smem, kt + 1 < nk ? c : cn, kt + 1 < nk ? kt + 1 : kt + 1 - nk, (g + 1) & 1, w, lane);
      if (STAGE == 2 && kt == nk - kAhead && !idle) {  // the epilogue's first inputs
        const E ep(args, args.mats + tl.mat, c, wm, wn, lane);
#pragma unroll
        for (int b = 0; b < kDepth; ++b) ep.load(b, in[b % E::kInSlots]);
      }
      if (STAGE == 3 && kt == nk - 1) {  // the next tile's diagonal words, before its second slab
        if (kLoIn)
          resn = issue_res_regs(cn, cn.i0 + 128 * wm, lane);
        else
          issue_res_lds(res_lds(smem, half ^ 1, w), cn, cn.i0 + 128 * wm, lane);
      }
      const int slot = (g + kAhead) % G::kRing;
      if (kt + kAhead < nk)
        issue_slab<STAGE>(smem, c, kt + kAhead, slot, w, lane);
      else
        issue_slab<STAGE>(smem, cn, kt + kAhead - nk, slot, w, lane);
      if (STAGE == 2 && kt >= nk - kAhead) vm_pre += kD;
      const char* s = smem + (g % G::kRing) * G::kSlot;
      if (!idle) {
        const char* p = c.psrc ? s + (c.psrc - 1) * kHalf : s + G::kPOff;
        if (STAGE == 3) {
          const int rel = kt * kBK - R0;  // this slab's K rows are output rows of the wave
          if (rel >= 0 && rel < 128) {
            const char* lo = smem + kLoBase + (g & 1) * kLoBuf;
            const float al = alpha + (kLoIn ? res_of(res, rel >> 5) : read_res(res_lds(smem, half, w), lane, rel >> 5));
            switch (rel >> 5) {
              case 0: fold_x<kLoIn>(acc[0], p, lo, wn, lane, al); break;
              case 1: fold_x<kLoIn>(acc[1], p, lo, wn, lane, al); break;
              case 2: fold_x<kLoIn>(acc[2 % G::kMI], p, lo, wn, lane, al); break;
              default: fold_x<kLoIn>(acc[3 % G::kMI], p, lo, wn, lane, al); break;
            }
          }
          mma_slab<true, G::kMI>(acc, s + wm * kHalf, p, wn, lane, fo);
        } else {
          mma_slab<false, G::kMI>(acc, s + wm * (G::kWide ? kHalf : kHalf / 2), p, wn, lane, fo);
        }
      }
      ++g;
    }

    // epilogue: the last slab's slot holds the waves' staged blocks
    MUON_LDS_BARRIER();  // all waves are done with the last slab
    pend = 0;
    if (!idle) {
      const E ep(args, args.mats + tl.mat, c, wm, wn, lane);
      int early_w = 0;  // requests made after the next tile's first slabs, before run()
      if (E::kLastIt) {  // the weight step requests its first W blocks here (registers are short in the loop)
#pragma unroll
        for (int b = 0; b < kDepth; ++b) ep.load(b, in[b % E::kInSlots]);
        vm_pre = 0;
        early_w = kDepth * ep.loads_per_block();
      }
      Stage st;
      st.base = smem + ((g + G::kRing - 1) % G::kRing) * G::kSlot + w * kBlock;
      pend = early_w + ep.run(acc, st, in, vm_pre);
    }
    if (!more) break;
    q = qn;
    tl = tn;
    c = cn;
    res = resn;
    half ^= 1;
  }
}

// ---------------------------------------------------------- fused launch --
//
// One persistent launch runs every bf16 product of a step.  The planner puts
// each matrix, with all of its tiles, on one XCD; XCD x's queue is one
// iteration's tiles of its matrices (Gram, then polynomial, then update),
// repeated T times.  A block reads the XCD it runs on from the hardware, takes
// the next entry of that XCD's queue (an atomic counter), waits until the
// tiles the entry reads are finished, runs the tile and counts it finished in
// its matrix's counter.  Tile (t, product) of a matrix reads what the
// previous product of iteration t (or the update of iteration t - 1) wrote,
// so it waits for the counter to reach the tiles of everything before it:
//   Gram t:    (t - 1) (ng + npl + nu)
//   poly t:    (t - 1) (ng + npl + nu) + ng
//   update t:  (t - 1) (ng + npl + nu) + ng + npl
// and that also orders every overwrite after the reads of the old contents
// (A, B and X's two copies are reused every iteration).
//
// Progress: entries are claimed in queue order and every wait is for entries
// earlier in the same queue, so the earliest unfinished entry is always
// either claimed by a running block whose waits are met or next to be
// claimed; no block ever waits for a block that is not running.  Each wait is
// still bounded: after spin_limit polls the block sets the status word and
// stops, and so does every block that sees the status set.
//
// Memory: producer and consumer of a matrix's data run on one XCD and share
// its L2.  A finished tile's stores are complete (vmcnt 0) before its counter
// moves; a block that waited invalidates at agent scope (buffer_inv sc1)
// before requesting the tile's operands: the group-scope form (sc0) left
// stale operand data visible on MI355X (results differed from the three-launch
// plan's), the agent-scope form makes them bitwise equal.

// Thread 0: wait until `dep` reaches `need` (true), or give up (false).
__device__ __noinline__ bool fused_wait(int32_t* dep, int need, int32_t* status, int limit) {
  for (int spins = 0;; ++spins) {
    if (__hip_atomic_load(dep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) return true;
    if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    if (spins >= limit) {
      __hip_atomic_fetch_or(status, (int)kFusedWaitGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// One tile of the fused launch, on its own: the ring starts empty and the
// tile's epilogue stores are complete when it returns.
template <int STAGE, int MODE>
__device__ __forceinline__ void fused_tile(const StageArgs& args, char* smem, const Tile& tl, int w, int wm, int wn,
                                           int lane, const FragOff& fo) {
  const Ctx c = ctx_of<STAGE, MODE>(args, tl);
  Ctx cn = c;
  cn.p = nullptr;  // no next tile: empty requests
  const u32x4 res = tile_prologue<STAGE, MODE>(smem, c, w, wm, lane);
  u32x4 resn;
  int g = 0;
  (void)tile_pass<STAGE, MODE>(args, smem, tl, c, cn, g, 0, w, wm, wn, lane, fo, res, resn, 0);
  MUON_WAIT_VMCNT(0);
}

__global__ __launch_bounds__(kThreads, kBlocks) void ns_fused_kernel(FusedArgs fa) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  volatile int32_t* ctl = (volatile int32_t*)smem;  // between tiles the LDS is free: claim and verdict
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int lane = threadIdx.x & 63;
  const FragOff fo = frag_off(lane);
  int hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(hw));
  const int x = hw & (kXcds - 1);
  const int per = fa.qlen[x];
  const int total = per * fa.T;
  const Tile* queue = fa.queue + fa.qoff[x];
  for (;;) {
    if (threadIdx.x == 0) {
      const bool stop = __hip_atomic_load(fa.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      ctl[0] = stop ? total : __hip_atomic_fetch_add(fa.heads + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    MUON_LDS_BARRIER();
    const int e = __builtin_amdgcn_readfirstlane(ctl[0]);
    if (e >= total) break;
    const int t = e / per + 1;
    const uint64_t raw = *(const MUON_CONST uint64_t*)(const void*)(queue + (e - (t - 1) * per));
    const Tile tl = tile_of(raw);
    const int stage = (int)(raw >> 48);  // Tile::pad: the product (tile_of leaves it out)
    const DevMat* m = fa.mats + tl.mat;
    int32_t* dep = load_uniform(&m->dep);
    {
      // the tile must lie inside its matrix (the epilogues' stores are not
      // bounds-checked): an entry that does not is reported, never run
      const int mp = load_uniform(&m->mp), np = load_uniform(&m->np);
      const int ti = tl.ti, tj = tl.tj;
      bool valid = dep != nullptr;
      if (stage == 1) valid = valid && ti <= tj && tj < mp / 128;
      else if (stage == 2) valid = valid && 2 * ti <= tj && tj < mp / 128;
      else if (stage == 3) valid = valid && ti < mp / 256 && tj < np / 128;
      else valid = false;
      if (!valid) {
        if (threadIdx.x == 0)
          __hip_atomic_fetch_or(fa.status, (int)kFusedBadEntry, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    if (threadIdx.x == 0) {
      const int ng = load_uniform(&m->ng), npl = load_uniform(&m->npl), nu = load_uniform(&m->nu);
      const int need = (t - 1) * (ng + npl + nu) + (stage >= 2 ? ng : 0) + (stage == 3 ? npl : 0) + fa.dep_bias;
      ctl[1] = fused_wait(dep, need, fa.status, fa.spin_limit) ? 1 : 0;
    }
    MUON_LDS_BARRIER();
    const int ok = __builtin_amdgcn_readfirstlane(ctl[1]);
    asm volatile("buffer_inv sc1" ::: "memory");
    MUON_LDS_BARRIER();  // every wave has read ctl before the tile's requests land over it
    if (!ok) break;
    StageArgs sa;
    sa.mats = fa.mats;
    sa.tiles = nullptr;
    sa.ntiles = 0;
    sa.t = t;
    sa.T = fa.T;
    sa.kmaster = fa.kmaster;
    sa.a = fa.coef[t - 1][0];
    sa.b = fa.coef[t - 1][1];
    sa.c = fa.coef[t - 1][2];
    sa.lr = fa.lr;
    if (stage == 1) {
      fused_tile<1, 0>(sa, smem, tl, w, wm, wn, lane, fo);
    } else if (stage == 2) {
      fused_tile<2, 0>(sa, smem, tl, w, wm, wn, lane, fo);
    } else {  // stage 3 (checked above)
      const bool last = t == fa.T, hilo = t <= fa.kmaster, write_lo = !last && t < fa.kmaster;
      if (last) {
        if (hilo)
          fused_tile<3, kHiLo | kLast>(sa, smem, tl, w, wm, wn, lane, fo);
        else
          fused_tile<3, kLast>(sa, smem, tl, w, wm, wn, lane, fo);
      } else if (write_lo) {
        fused_tile<3, kHiLo | kWriteLo>(sa, smem, tl, w, wm, wn, lane, fo);
      } else if (hilo) {
        fused_tile<3, kHiLo>(sa, smem, tl, w, wm, wn, lane, fo);
      } else {
        fused_tile<3, 0>(sa, smem, tl, w, wm, wn, lane, fo);
      }
    }
    MUON_BARRIER();  // every wave's stores are complete
    if (threadIdx.x == 0) __hip_atomic_fetch_add(dep, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

// ------------------------------------------------------------ launchers --
#define MUON_BF16_KERNEL(S, M) ((const void*)ns_bf16_kernel<S, M>)

hipError_t prepare_bf16_kernels() {
  const void* fns[] = {MUON_BF16_KERNEL(1, 0), MUON_BF16_KERNEL(2, 0), MUON_BF16_KERNEL(3, 0),
                       MUON_BF16_KERNEL(3, 1), MUON_BF16_KERNEL(3, 5), MUON_BF16_KERNEL(3, 2),
                       MUON_BF16_KERNEL(3, 3), (const void*)ns_fused_kernel};
  for (const void* f : fns) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static hipError_t launch_bf16(const void* fn, int blocks, const StageArgs& args, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
  void* kargs[] = {(void*)&args};
  return hipExtLaunchKernel(fn, dim3(blocks), dim3(kThreads), kargs, kLds, stream, ev0, ev1, 0);
}

hipError_t launch_fused(const FusedArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  void* kargs[] = {(void*)&args};
  return hipExtLaunchKernel((const void*)ns_fused_kernel, dim3(blocks), dim3(kThreads), kargs, kLds, stream, ev0, ev1,
                            0);
}

hipError_t launch_stage_bf16(int stage, const StageArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0,
                             hipEvent_t ev1) {
  const bool last = args.t == args.T;
  const bool hilo = args.t <= args.kmaster;
  const bool write_lo = !last && args.t < args.kmaster;
  const void* fn = nullptr;
  if (stage == 1) fn = MUON_BF16_KERNEL(1, 0);
  if (stage == 2) fn = MUON_BF16_KERNEL(2, 0);
  if (stage == 3) {
    if (last)
      fn = hilo ? MUON_BF16_KERNEL(3, 3) : MUON_BF16_KERNEL(3, 2);
    else if (write_lo)
      fn = MUON_BF16_KERNEL(3, 5);
    else
      fn = hilo ? MUON_BF16_KERNEL(3, 1) : MUON_BF16_KERNEL(3, 0);
  }
  if (!fn) return hipErrorInvalidValue;
  return launch_bf16(fn, blocks, args, stream, ev0, ev1);
}

}  // namespace muon
