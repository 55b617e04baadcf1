// Internal layout shared by the host planner and the gfx950 kernels.
//
// Every matrix is handled in its canonical orientation X (m x n, m <= n):
// X = U when rows <= cols, X = U^T otherwise.  All workspace buffers of a
// matrix are padded to whole NS tiles (multiples of kTile in both
// dimensions).  The padding is zero in X0 (the momentum kernel writes it) and
// the iteration keeps it zero exactly (zero rows/columns stay zero under
// X X^T, b A + c A A and a X + B X), so the product kernels need no bounds
// checks; only the final weight step looks at the true extents.
#pragma once

#include <stdint.h>

namespace muon {

constexpr int kTile = 128;     // NS product tile edge (fp32 products; columns of bf16 tiles)
constexpr int kTileRowsBf16 = 256;  // rows of a bf16 product tile (X, A, B padded to multiples of it)
constexpr int kMomTile = 64;   // momentum kernel tile edge
constexpr int kThreads = 256;  // threads per block, every kernel
constexpr int kXcds = 8;       // MI355X: 8 XCDs, blocks dispatched round-robin
constexpr uint16_t kNullMat = 0xFFFF;  // tile-table filler: the block exits
constexpr double kEps = 1e-7;
// On the bf16 path, matrices whose short side is below this run the fp32
// arithmetic: with few terms in the A*A and B*X contractions the bf16 operand
// rounding averages out less (4x8 inputs reach 2-5e-2 relative error in bf16,
// short sides of 64 up to 1.8e-2 on MI355X, 128 and more at most 1.4e-2),
// while their cost is negligible.
constexpr int kMinBf16Side = 128;

// One matrix, as the kernels see it.
struct DevMat {
  void* w;            // weights (rows x cols), f32 or bf16
  const void* g;      // gradient (rows x cols), f32 or bf16
  float* mom;         // momentum (rows x cols), f32
  uint8_t* xlo;       // bf16 path: low byte of X (the rounded fp32-pattern distance to bf16(X) / 256, mp x np); else null
  void* xo[2];        // operand copies of X (ping-pong), bf16 or f32, mp x np
  void* a;            // A = X X^T, mp x mp (bf16 or f32)
  void* b;            // B = b A + c A A, mp x mp; on the bf16 path followed directly by mp fp32 words,
                      // for each row i what B's stored diagonal lacks: the change of B_ii that the
                      // rounding of A_ii causes (stored by the Gram kernel), plus B_ii - bf16(B_ii)
                      // (added by the polynomial kernel)
  float* part;        // momentum-kernel partial sums of squares, one per tile
  float* sc;          // [0] = 1/(||U||_F + eps), [1] = ||U||_F
  int32_t rows, cols; // original shape
  int32_t m, n;       // canonical shape (m <= n)
  int32_t mp, np;     // padded canonical shape
  int32_t transposed; // rows > cols
  int32_t w_bf16;     // weight dtype is bf16
  int32_t g_bf16;     // gradient dtype is bf16
  int32_t nparts;     // number of momentum tiles (= partial sums)
  int32_t mom_tiles_n;// momentum tiles along the canonical n axis
  float scale;        // s of the weight step (already defaulted to 1)
  int32_t vec_g;      // gradient and momentum rows can be read 8 elements at a time
  int32_t vec_w;      // weight rows can be read/written 4 elements at a time
  int32_t f32;        // this matrix's products use fp32 operands (xo, a, b are fp32)
  int32_t pad_;
  // fused launch (bf16 matrices of a fused plan; null / 0 otherwise)
  int32_t* dep;       // tiles of this matrix finished in the current step
  int32_t* heads;     // set on the first matrix only: the fused launch's claim counters, zeroed with dep
  int32_t ng, npl, nu;// the matrix's Gram, polynomial and update tiles per iteration
  int32_t pad2_;
};

struct Tile {
  uint16_t mat;  // matrix index, kNullMat for filler
  uint16_t ti;   // tile row
  uint16_t tj;   // tile column
  uint16_t pad;
};

struct StageArgs {
  const DevMat* mats;
  const Tile* tiles;
  int32_t ntiles;   // table length (persistent blocks stride through it)
  int32_t t;        // iteration, 1-based
  int32_t T;        // iterations this step
  int32_t kmaster;  // bf16 path: iterations 1..kmaster read X as its (bf16, low byte) pair in a*X
  float a, b, c;
  float lr;
};

// The fused launch: every bf16 product of a step in one persistent launch.
// XCD x works through its queue, one iteration's tiles (Gram, then
// polynomial, then update, of the matrices placed on it) repeated T times;
// blocks claim the next entry from heads[x] and wait until the tiles it reads
// are finished (per-matrix counters in DevMat::dep).
constexpr int kFusedMaxT = 16;  // iterations whose coefficients fit the launch arguments
enum { kFusedWaitGaveUp = 1, kFusedBadEntry = 2 };  // FusedArgs::status bits
struct FusedArgs {
  const DevMat* mats;
  const Tile* queue;            // Tile::pad = product (1 Gram, 2 polynomial, 3 update)
  int32_t qoff[kXcds];          // XCD x: one iteration's entries at queue[qoff[x] .. qoff[x] + qlen[x])
  int32_t qlen[kXcds];
  int32_t* heads;               // [kXcds] entries claimed so far this step
  int32_t* status;              // 0, or why a block gave up (sticky until read)
  int32_t T, kmaster;
  float coef[kFusedMaxT][3];    // (a, b, c) of iteration t at coef[t - 1]
  float lr;
  int32_t spin_limit;           // polls of one dependency wait before it gives up
  int32_t dep_bias;             // added to every wait's target (0; a test of the give-up path raises it)
  int32_t pad_;
};

struct MomArgs {
  const DevMat* mats;
  const Tile* tiles;
  float mu;
  int32_t nesterov;
};

struct ApplyArgs {
  const DevMat* mats;
  const Tile* tiles;
  float lr;
};

}  // namespace muon
