// Host side of the Muon C ABI: validation, planning, workspace layout,
// launch sequence and per-launch timing.  See include/muon.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "muon_internal.h"

namespace muon {
hipError_t launch_momentum(const MomArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_apply(const ApplyArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_stage(int stage, bool f32, const StageArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0,
                        hipEvent_t ev1);
hipError_t prepare_stage_kernels();
hipError_t launch_stage_bf16(int stage, const StageArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0,
                             hipEvent_t ev1);
hipError_t prepare_bf16_kernels();
hipError_t launch_fused(const FusedArgs& args, int blocks, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_norm(const DevMat* mats, int n, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
}  // namespace muon

using namespace muon;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MUON_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

void release(muon_plan* p);

constexpr int kSlots = 8;           // device copies of the matrix table (pointer updates)
constexpr size_t kAlign = 256;
constexpr int kMaxMatrices = 65000; // tile tables index matrices with 16 bits
constexpr int64_t kMaxDim = 1 << 20;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// The launches of each matrix group (contiguous runs of matrices of about
// equal Newton-Schulz cost) go to a stream of their own: each group's kernels
// fill the others' launch gaps and end-of-launch tails.
constexpr int kGroups = 4;  // at most; options.groups selects how many are used

struct Options {
  int path = MUON_PATH_BF16;
  int kmaster = 3;
  int zero = 0;
  int maxT = 64;
  int groups = 2;
  int fused = 0;
};

int read_options(const muon_options* o, Options* out) {
  Options r;
  if (o) {
    if (o->path != MUON_PATH_BF16 && o->path != MUON_PATH_F32)
      return fail(MUON_E_UNSUPPORTED, "options.path %d is not MUON_PATH_BF16 or MUON_PATH_F32", o->path);
    r.path = o->path;
    r.kmaster = o->x_master_iters < 0 ? 3 : o->x_master_iters;
    r.zero = o->zero_momentum;
    r.maxT = o->max_T <= 0 ? 64 : o->max_T;
    r.groups = o->groups <= 0 ? 2 : o->groups;
    if (r.groups > kGroups) return fail(MUON_E_INVAL, "options.groups %d exceeds %d", r.groups, kGroups);
    r.fused = o->fused != 0;
    if (r.fused) r.groups = 1;  // a fused plan runs on the caller's stream
    if (r.maxT > 4096) return fail(MUON_E_INVAL, "options.max_T %d exceeds 4096", r.maxT);
    if (r.kmaster > 4096) return fail(MUON_E_INVAL, "options.x_master_iters %d exceeds 4096", r.kmaster);
  }
  if (r.path == MUON_PATH_F32) r.kmaster = 0;
  *out = r;
  return MUON_OK;
}

// Shape/dtype check of one descriptor.  `need_ptrs`: pointers must be set.
int check_desc(const muon_matrix_desc& d, int idx, bool need_ptrs) {
  if (d.rows <= 0 || d.cols <= 0)
    return fail(MUON_E_INVAL, "matrix %d: rows=%lld cols=%lld must be positive", idx, (long long)d.rows,
                (long long)d.cols);
  if (d.rows > kMaxDim || d.cols > kMaxDim)
    return fail(MUON_E_INVAL, "matrix %d: %lld x %lld exceeds the %lld limit per side", idx, (long long)d.rows,
                (long long)d.cols, (long long)kMaxDim);
  if (d.ld_w != 0 && d.ld_w != d.cols)
    return fail(MUON_E_UNSUPPORTED, "matrix %d: ld_w=%lld must equal cols=%lld", idx, (long long)d.ld_w,
                (long long)d.cols);
  if (d.ld_g != 0 && d.ld_g != d.cols)
    return fail(MUON_E_UNSUPPORTED, "matrix %d: ld_g=%lld must equal cols=%lld", idx, (long long)d.ld_g,
                (long long)d.cols);
  if (d.g_dtype != MUON_DTYPE_BF16 && d.g_dtype != MUON_DTYPE_F32)
    return fail(MUON_E_UNSUPPORTED, "matrix %d: g_dtype %d unsupported", idx, d.g_dtype);
  if (d.w_dtype != MUON_DTYPE_BF16 && d.w_dtype != MUON_DTYPE_F32)
    return fail(MUON_E_UNSUPPORTED, "matrix %d: w_dtype %d unsupported", idx, d.w_dtype);
  if (d.reserved != 0) return fail(MUON_E_INVAL, "matrix %d: reserved field must be 0", idx);
  if (!std::isfinite(d.scale)) return fail(MUON_E_INVAL, "matrix %d: scale is not finite", idx);
  // the kernels address each matrix's buffers with 32-bit byte offsets
  const int64_t mp = round_up(std::min(d.rows, d.cols), kTileRowsBf16), np = round_up(std::max(d.rows, d.cols), kTile);
  if (mp * np * 4 >= (int64_t(1) << 31) || d.rows * d.cols * 4 >= (int64_t(1) << 31))
    return fail(MUON_E_UNSUPPORTED, "matrix %d: %lld x %lld needs more than 2 GiB per buffer", idx,
                (long long)d.rows, (long long)d.cols);
  if (need_ptrs) {
    if (!d.weight || !d.grad || !d.momentum) return fail(MUON_E_INVAL, "matrix %d: null device pointer", idx);
    if (d.weight == d.grad || d.weight == (void*)d.momentum || d.grad == (const void*)d.momentum)
      return fail(MUON_E_INVAL, "matrix %d: weight, grad and momentum must be distinct buffers", idx);
    const size_t wal = d.w_dtype == MUON_DTYPE_F32 ? 4 : 2, gal = d.g_dtype == MUON_DTYPE_F32 ? 4 : 2;
    if ((uintptr_t)d.weight % wal || (uintptr_t)d.grad % gal || (uintptr_t)d.momentum % 4)
      return fail(MUON_E_INVAL, "matrix %d: pointer not aligned to its element size", idx);
  }
  return MUON_OK;
}


struct Layout {
  // per matrix byte offsets into the workspace
  struct M {
    size_t xlo, xo0, xo1, a, b, bres, part, sc;
  };
  std::vector<M> m;
  size_t slots = 0, slot_bytes = 0;
  size_t mom_tiles[kGroups] = {};
  size_t ns_tiles[kGroups][2][3] = {};
  size_t fq = 0;    // fused plans: the XCD queues
  size_t fctl = 0;  // fused plans: claim counters [kXcds], then the status word
  size_t fdep = 0;  // fused plans: one finished-tile counter per matrix
  size_t total = 0;
};

struct Geometry {
  int rows, cols, m, n, mp, np, tr, nparts, mom_n, f32;
};

Geometry geometry(const muon_matrix_desc& d, int path) {
  Geometry g;
  g.rows = (int)d.rows;
  g.cols = (int)d.cols;
  g.tr = d.rows > d.cols;
  g.m = (int)std::min(d.rows, d.cols);
  g.n = (int)std::max(d.rows, d.cols);
  g.f32 = path == MUON_PATH_F32 || g.m < kMinBf16Side;
  // bf16 products run 256 x 128 tiles (rows of X, A, B in 256-row panels),
  // fp32 products 128 x 128 tiles
  g.mp = (int)round_up(g.m, g.f32 ? kTile : kTileRowsBf16);
  g.np = (int)round_up(g.n, kTile);
  g.mom_n = g.np / kMomTile;
  g.nparts = (g.mp / kMomTile) * g.mom_n;
  return g;
}

// Tile lists: the momentum list covers every matrix; the product lists are
// split by operand precision (index 0: bf16 matrices, 1: fp32 matrices),
// since each launch runs one precision.
enum { kGram = 0, kPoly = 1, kUpd = 2 };
struct Tables {
  std::vector<Tile> mom[kGroups];       // [group]: momentum / apply tiles
  std::vector<Tile> ns[kGroups][2][3];  // [group][precision][kind]
  int first[kGroups + 1] = {};          // group g holds matrices first[g] .. first[g+1]-1
  // fused plans: one iteration's bf16 tiles per XCD (Tile::pad = product 1-3)
  std::vector<Tile> fq;                 // XCD by XCD
  int32_t qoff[kXcds] = {}, qlen[kXcds] = {};
  std::vector<int> fxcd;                // per matrix: its XCD, -1 when not in the fused launch
  std::vector<int32_t> fcount[3];       // per matrix: its Gram, polynomial and update tiles per iteration
};

// Product launches run kXcds * kBlocksPerXcd blocks (two resident blocks on
// each of the 32 CUs of an XCD), and block b takes table entries b, b + 512,
// b + 1024, ...  The tables are laid out for that stride.
constexpr int kBlocksPerXcd = 64;
constexpr int kProductGrid = kXcds * kBlocksPerXcd;

// Tiles of one kind, ordered for the MI355X dispatcher, which places block b
// on XCD b % 8.  The tiles of each cost class are listed matrix by matrix and
// cut into 8 contiguous runs of equal total cost; XCD x gets run x of every
// class, most expensive class first.  Each XCD therefore works on few
// matrices at a time (they stay in its L2) and the XCDs get equal work.
// Inside a run, each tile in turn goes to the block with the least work so far
// (longest tiles first, ties to the lowest block), the schedule the blocks
// would reach if each took the next tile when it finished.  Block j of XCD x
// (block index 8j + x) finds its r-th tile at entry 8(r * kBlocksPerXcd + j) + x;
// entries of blocks with fewer tiles hold null tiles that exit at once.
struct CostTile {
  Tile t;
  double cost;  // work of this tile (128 x 128 x 128 units)
};
std::vector<Tile> xcd_order(const std::vector<std::vector<CostTile>>& per_mat, const std::vector<double>& tile_cost) {
  const int nm = (int)per_mat.size();
  std::vector<int> order(nm);
  for (int i = 0; i < nm; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return tile_cost[x] > tile_cost[y]; });
  std::vector<std::vector<CostTile>> runs(kXcds);
  // one cost class (matrices whose tiles cost the same) at a time, so that
  // every XCD gets its share of long and of short tiles
  for (size_t c0 = 0; c0 < order.size();) {
    size_t c1 = c0;
    double total = 0.0;
    while (c1 < order.size() && tile_cost[order[c1]] == tile_cost[order[c0]]) {
      for (const CostTile& t : per_mat[order[c1]]) total += t.cost;
      ++c1;
    }
    double acc = 0.0;
    for (size_t q = c0; q < c1 && total > 0.0; ++q) {
      const int i = order[q];
      for (const CostTile& t : per_mat[i]) {
        // the run whose cost share contains the midpoint of this tile
        int x = (int)((acc + 0.5 * t.cost) * kXcds / total);
        x = std::min(std::max(x, 0), kXcds - 1);
        runs[x].push_back(t);
        acc += t.cost;
      }
    }
    c0 = c1;
  }
  // per XCD: the tiles of each block, in the order the block runs them
  std::vector<std::vector<Tile>> blk((size_t)kXcds * kBlocksPerXcd);
  size_t rounds = 0;
  for (int x = 0; x < kXcds; ++x) {
    std::vector<double> load(kBlocksPerXcd, 0.0);
    for (const CostTile& t : runs[x]) {
      const int j = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      load[j] += t.cost;
      std::vector<Tile>& l = blk[(size_t)x * kBlocksPerXcd + j];
      l.push_back(t.t);
      rounds = std::max(rounds, l.size());
    }
  }
  std::vector<Tile> out(rounds * kProductGrid, Tile{kNullMat, 0, 0, 0});
  for (int x = 0; x < kXcds; ++x)
    for (int j = 0; j < kBlocksPerXcd; ++j) {
      const std::vector<Tile>& l = blk[(size_t)x * kBlocksPerXcd + j];
      for (size_t r = 0; r < l.size(); ++r) out[(r * kBlocksPerXcd + j) * kXcds + x] = l[r];
    }
  while (!out.empty() && out.back().mat == kNullMat) out.pop_back();
  return out;
}

// Group g holds matrices [first[g], first[g + 1]): contiguous runs of about
// equal Newton-Schulz cost, boundary g where the running cost is closest to
// g / groups of the total (groups beyond the matrix count stay empty).
void group_bounds(const std::vector<Geometry>& geo, int groups, int (&first)[kGroups + 1]) {
  const int nm = (int)geo.size();
  std::vector<double> pre(nm + 1, 0.0);
  for (int i = 0; i < nm; ++i) {
    const double m = geo[i].mp, n = geo[i].np;
    pre[i + 1] = pre[i] + m * m * (2.0 * n + m);
  }
  first[0] = 0;
  for (int g = 1; g <= kGroups; ++g) {
    if (g >= groups) {
      first[g] = nm;
      continue;
    }
    const double target = pre[nm] * g / groups;
    int best = first[g - 1];
    for (int s = first[g - 1]; s <= nm; ++s)
      if (std::fabs(pre[s] - target) < std::fabs(pre[best] - target)) best = s;
    first[g] = best;
  }
}

// A bf16 matrix's product tiles, each with its cost.  The Gram product takes
// 128 x 128 tiles on or above the diagonal (a diagonal tile costs a full one:
// its idle wave keeps pace with the others through the slab barriers).  The
// polynomial and the update take 256 x 128 tiles (row panel a of 256 rows,
// column panel b of 128); the polynomial's are those reaching the upper
// triangle at 128 granularity, b >= 2a, and when b == 2a rows 128..255 lie
// below it.  Update tiles go column panel by column panel: the tiles of one X
// column panel run together and share it in L2.
void bf16_tiles(const Geometry& g, int i, std::vector<CostTile>& gram, std::vector<CostTile>& poly,
                std::vector<CostTile>& upd) {
  const double K1 = g.np / 128.0, K2 = g.mp / 128.0;
  const int tm = g.mp / kTileRowsBf16, tc = g.mp / kTile, tn = g.np / kTile;
  for (int a = 0; a < tc; ++a)
    for (int b = a; b < tc; ++b) gram.push_back(CostTile{Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 1}, K1});
  for (int a = 0; a < tm; ++a)
    for (int b = 2 * a; b < tc; ++b)
      poly.push_back(CostTile{Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 2}, (b == 2 * a ? 1.0 : 2.0) * K2});
  for (int b = 0; b < tn; ++b)
    for (int a = 0; a < tm; ++a) upd.push_back(CostTile{Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 3}, 2.0 * K2});
}

// Fused plans: each bf16 matrix goes whole to one XCD, most expensive first,
// each to the XCD with the least work so far; XCD x's queue lists one
// iteration's tiles of its matrices, product by product (Gram, polynomial,
// update), matrix by matrix in placement order within a product.  A
// product's tiles of the first-placed matrices are therefore the first to
// have their inputs ready.
void build_fused(const std::vector<Geometry>& geo, Tables& t) {
  const int nm = (int)geo.size();
  t.fxcd.assign(nm, -1);
  for (int k = 0; k < 3; ++k) t.fcount[k].assign(nm, 0);
  std::vector<std::vector<CostTile>> tiles[3];
  for (int k = 0; k < 3; ++k) tiles[k].resize(nm);
  std::vector<double> cost(nm, 0.0);
  std::vector<int> order;
  for (int i = 0; i < nm; ++i) {
    if (geo[i].f32) continue;
    bf16_tiles(geo[i], i, tiles[0][i], tiles[1][i], tiles[2][i]);
    for (int k = 0; k < 3; ++k) {
      t.fcount[k][i] = (int32_t)tiles[k][i].size();
      for (const CostTile& c : tiles[k][i]) cost[i] += c.cost;
    }
    order.push_back(i);
  }
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return cost[x] > cost[y]; });
  double load[kXcds] = {};
  std::vector<int> on[kXcds];
  for (int i : order) {
    const int x = (int)(std::min_element(load, load + kXcds) - load);
    load[x] += cost[i];
    on[x].push_back(i);
    t.fxcd[i] = x;
  }
  t.fq.clear();
  for (int x = 0; x < kXcds; ++x) {
    t.qoff[x] = (int32_t)t.fq.size();
    for (int k = 0; k < 3; ++k)
      for (int i : on[x])
        for (const CostTile& c : tiles[k][i]) t.fq.push_back(c.t);
    t.qlen[x] = (int32_t)t.fq.size() - t.qoff[x];
  }
}

Tables build_tables(const std::vector<Geometry>& geo, int groups, bool fused) {
  Tables t;
  if (fused) build_fused(geo, t);
  const int nm = (int)geo.size();
  group_bounds(geo, groups, t.first);
  auto group_of = [&](int i) {
    int g = 0;
    while (i >= t.first[g + 1]) ++g;
    return g;
  };
  for (int grp = 0; grp < kGroups; ++grp)
  for (int prec = 0; prec < 2; ++prec) {
    std::vector<std::vector<CostTile>> gram(nm), poly(nm), upd(nm);
    std::vector<double> gram_k(nm), poly_k(nm), upd_k(nm);  // cost classes: K of the tiles
    for (int i = 0; i < nm; ++i) {
      const Geometry& g = geo[i];
      if (g.f32 != prec || group_of(i) != grp) continue;
      const double K1 = g.np / 128.0, K2 = g.mp / 128.0;
      if (prec == 0) {
        bf16_tiles(g, i, gram[i], poly[i], upd[i]);
      } else {
        // fp32: 128 x 128 tiles, upper triangle of the symmetric products
        const int tm = g.mp / kTile, tn = g.np / kTile;
        for (int a = 0; a < tm; ++a)
          for (int b = a; b < tm; ++b) {
            gram[i].push_back(CostTile{Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 0}, K1});
            poly[i].push_back(CostTile{Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 0}, K2});
          }
        for (int b = 0; b < tn; ++b)
          for (int a = 0; a < tm; ++a) upd[i].push_back(CostTile{Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 0}, K2});
      }
      gram_k[i] = K1;
      poly_k[i] = K2;
      upd_k[i] = K2;
    }
    t.ns[grp][prec][kGram] = xcd_order(gram, gram_k);
    t.ns[grp][prec][kPoly] = xcd_order(poly, poly_k);
    t.ns[grp][prec][kUpd] = xcd_order(upd, upd_k);
  }
  for (int i = 0; i < nm; ++i) {
    const Geometry& g = geo[i];
    std::vector<Tile>& mom = t.mom[group_of(i)];
    for (int a = 0; a < g.mp / kMomTile; ++a)
      for (int b = 0; b < g.np / kMomTile; ++b) mom.push_back(Tile{(uint16_t)i, (uint16_t)a, (uint16_t)b, 0});
  }
  return t;
}

size_t layout(const std::vector<Geometry>& geo, const Options& o, const Tables& t, Layout* L) {
  const int nm = (int)geo.size();
  size_t off = 0;
  L->slot_bytes = align_up(sizeof(DevMat) * nm, kAlign);
  L->slots = off;
  off += L->slot_bytes * kSlots;
  for (int grp = 0; grp < kGroups; ++grp) {
    L->mom_tiles[grp] = off;
    off = align_up(off + sizeof(Tile) * t.mom[grp].size(), kAlign);
  }
  for (int grp = 0; grp < kGroups; ++grp)
    for (int prec = 0; prec < 2; ++prec)
      for (int k = 0; k < 3; ++k) {
        L->ns_tiles[grp][prec][k] = off;
        off = align_up(off + sizeof(Tile) * t.ns[grp][prec][k].size(), kAlign);
      }
  if (!t.fq.empty()) {
    L->fq = off;
    off = align_up(off + sizeof(Tile) * t.fq.size(), kAlign);
    L->fctl = off;
    off = align_up(off + sizeof(int32_t) * (kXcds + 1), kAlign);
    L->fdep = off;
    off = align_up(off + sizeof(int32_t) * nm, kAlign);
  }
  L->m.resize(nm);
  for (int i = 0; i < nm; ++i) {
    const Geometry& g = geo[i];
    const size_t es = g.f32 ? 4 : 2;
    const size_t xe = (size_t)g.mp * g.np, ae = (size_t)g.mp * g.mp;
    Layout::M& m = L->m[i];
    m.xlo = (size_t)-1;
    if (!g.f32 && o.kmaster > 0) {
      m.xlo = off;
      off = align_up(off + xe, kAlign);  // one low byte per element
    }
    m.xo0 = off;
    off = align_up(off + xe * es, kAlign);
    m.xo1 = off;
    off = align_up(off + xe * es, kAlign);
    m.a = off;
    off = align_up(off + ae * es, kAlign);
    // bf16 path: B is followed directly by mp fp32 words, what B's stored
    // diagonal lacks (the kernels reach them through B's buffer resource)
    m.b = off;
    off = align_up(off + ae * es + (g.f32 ? 0 : sizeof(float) * g.mp), kAlign);
    m.bres = g.f32 ? (size_t)-1 : m.b + ae * es;
    m.part = off;
    off = align_up(off + sizeof(float) * g.nparts, kAlign);
    m.sc = off;
    off = align_up(off + 4 * sizeof(float), kAlign);
  }
  L->total = off;
  return off;
}

int validate_all(const muon_matrix_desc* d, int n, bool need_ptrs) {
  if (!d) return fail(MUON_E_INVAL, "descriptor array is NULL");
  if (n <= 0 || n > kMaxMatrices) return fail(MUON_E_INVAL, "matrix count %d outside [1, %d]", n, kMaxMatrices);
  for (int i = 0; i < n; ++i) {
    int rc = check_desc(d[i], i, need_ptrs);
    if (rc) return rc;
  }
  return MUON_OK;
}

}  // namespace

struct muon_plan {
  int n = 0;
  Options opt;
  std::vector<Geometry> geo;
  std::vector<muon_matrix_desc> desc;  // shapes, dtypes, scales and current pointers
  Tables tab;
  Layout lay;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<DevMat> hmat;            // host image of the current table
  DevMat* host_slots[kSlots] = {};     // pinned staging, one per device slot
  hipEvent_t slot_ev[kSlots] = {};
  bool slot_used[kSlots] = {};
  int slot = 0;
  bool captured = false;  // a step of this plan was enqueued into a capturing stream
  int32_t spin_limit = 1 << 24;  // fused launch: polls of one dependency wait before it gives up
  int32_t dep_bias = 0;          // fused launch: added to every wait's target (tests only)
  hipEvent_t last_ev = nullptr;        // recorded after the last enqueued work
  bool last_valid = false;
  hipStream_t gs[kGroups] = {};        // the groups' Newton-Schulz streams (default priority)
  hipEvent_t fork_ev = nullptr, join_ev[kGroups] = {};
  // profiling
  bool prof = false;
  std::vector<hipEvent_t> pev;         // pairs: start, stop
  uint32_t pmask = ~0u;                // kinds whose launches are timed
  std::vector<int> pkind;              // kind of each pair
  size_t pused = 0;
  double pms[MUON_KIND_COUNT] = {};
  int64_t pcnt[MUON_KIND_COUNT] = {};
};

namespace {

DevMat make_devmat(const muon_plan* p, int i) {
  const Geometry& g = p->geo[i];
  const muon_matrix_desc& d = p->desc[i];
  const Layout::M& m = p->lay.m[i];
  DevMat r;
  std::memset(&r, 0, sizeof(r));
  r.w = d.weight;
  r.g = d.grad;
  r.mom = d.momentum;
  r.xlo = m.xlo == (size_t)-1 ? nullptr : (uint8_t*)(p->ws + m.xlo);
  r.xo[0] = p->ws + m.xo0;
  r.xo[1] = p->ws + m.xo1;
  r.a = p->ws + m.a;
  r.b = p->ws + m.b;
  r.part = (float*)(p->ws + m.part);
  r.sc = (float*)(p->ws + m.sc);
  r.rows = g.rows;
  r.cols = g.cols;
  r.m = g.m;
  r.n = g.n;
  r.mp = g.mp;
  r.np = g.np;
  r.transposed = g.tr;
  r.w_bf16 = d.w_dtype == MUON_DTYPE_BF16;
  r.g_bf16 = d.g_dtype == MUON_DTYPE_BF16;
  r.nparts = g.nparts;
  r.mom_tiles_n = g.mom_n;
  r.scale = d.scale > 0.f ? d.scale : 1.f;
  r.vec_g = (g.cols % 8 == 0) && ((uintptr_t)d.grad % 16 == 0) && ((uintptr_t)d.momentum % 16 == 0);
  r.vec_w = (g.cols % 4 == 0) && ((uintptr_t)d.weight % 16 == 0);
  r.f32 = g.f32;
  const Tables& t = p->tab;
  if (!t.fq.empty()) {
    if (t.fxcd[i] >= 0) {
      r.dep = (int32_t*)(p->ws + p->lay.fdep) + i;
      r.ng = t.fcount[0][i];
      r.npl = t.fcount[1][i];
      r.nu = t.fcount[2][i];
    }
    if (i == 0) r.heads = (int32_t*)(p->ws + p->lay.fctl);  // the norm launch zeroes them with matrix 0's block
  }
  return r;
}

DevMat* slot_ptr(const muon_plan* p, int s) { return (DevMat*)(p->ws + p->lay.slots + p->lay.slot_bytes * s); }

// Upload the host image of the matrix table into the next device slot.
int upload_table(muon_plan* p, hipStream_t stream) {
  const int s = (p->slot + 1) % kSlots;
  if (p->slot_used[s]) {
    hipError_t e = hipEventSynchronize(p->slot_ev[s]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(table slot)");
  }
  std::memcpy(p->host_slots[s], p->hmat.data(), sizeof(DevMat) * p->n);
  hipError_t e = hipMemcpyAsync(slot_ptr(p, s), p->host_slots[s], sizeof(DevMat) * p->n, hipMemcpyHostToDevice,
                                stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(matrix table)");
  p->slot = s;
  return MUON_OK;
}

int note_slot_use(muon_plan* p, hipStream_t stream) {
  hipError_t e = hipEventRecord(p->slot_ev[p->slot], stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(table slot)");
  p->slot_used[p->slot] = true;
  e = hipEventRecord(p->last_ev, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  p->last_valid = true;
  return MUON_OK;
}

// The event pair that times one launch, or null events when the launch is not
// profiled.  The launch records them itself (they take the dispatch's own
// start and end times), so profiling adds nothing to the stream.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

int prof_events(muon_plan* p, int kind, LaunchEvents* ev) {
  *ev = LaunchEvents{};
  if (!p->prof || !((p->pmask >> kind) & 1u)) return MUON_OK;
  if (p->pused * 2 + 2 > p->pev.size()) {
    for (int k = 0; k < 64; ++k) {
      hipEvent_t e;
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
      p->pev.push_back(e);
    }
  }
  const size_t idx = p->pused++;
  if (p->pkind.size() < p->pused) p->pkind.resize(p->pused);
  p->pkind[idx] = kind;
  ev->start = p->pev[2 * idx];
  ev->stop = p->pev[2 * idx + 1];
  return MUON_OK;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  return MUON_OK;
}

}  // namespace

extern "C" {

const char* muon_version(void) { return "muon-mi355x 1.0.0 (gfx950)"; }

const char* muon_last_error(void) { return g_err.c_str(); }

size_t muon_workspace_size(const muon_matrix_desc* descs, int n, const muon_options* opts) {
  Options o;
  if (read_options(opts, &o)) return 0;
  if (validate_all(descs, n, false)) return 0;
  std::vector<Geometry> geo(n);
  for (int i = 0; i < n; ++i) geo[i] = geometry(descs[i], o.path);
  Tables t = build_tables(geo, o.groups, o.fused);
  Layout L;
  return layout(geo, o, t, &L);
}

// All launches of one product kind, table after table, each padded with null
// tiles to a multiple of 8 so that entry b of the result still runs on XCD b % 8.
static std::vector<Tile> concat_tables(const Tables& t, int k) {
  std::vector<Tile> v;
  for (int grp = 0; grp < kGroups; ++grp)
    for (int prec = 0; prec < 2; ++prec) {
      const std::vector<Tile>& s = t.ns[grp][prec][k];
      if (s.empty()) continue;
      if (!v.empty()) v.resize((v.size() + kXcds - 1) / kXcds * kXcds, Tile{kNullMat, 0, 0, 0});
      v.insert(v.end(), s.begin(), s.end());
    }
  return v;
}

int muon_describe(const muon_matrix_desc* descs, int n, const muon_options* opts, muon_plan_info* info, int kind,
                  int32_t* tiles, int tile_cap, int32_t* n_tiles) {
  g_err.clear();
  Options o;
  int rc = read_options(opts, &o);
  if (rc) return rc;
  rc = validate_all(descs, n, false);
  if (rc) return rc;
  std::vector<Geometry> geo(n);
  for (int i = 0; i < n; ++i) geo[i] = geometry(descs[i], o.path);
  Tables t = build_tables(geo, o.groups, o.fused);
  Layout L;
  const size_t total = layout(geo, o, t, &L);
  if (info) {
    info->workspace_bytes = (int64_t)total;
    info->n_matrices = n;
    info->tile = kTile;
    info->bf16_tile_rows = kTileRowsBf16;
    info->bf16_tile_cols = kTile;
    size_t nmom = 0;
    for (int grp = 0; grp < kGroups; ++grp) nmom += t.mom[grp].size();
    info->blocks[MUON_KIND_MOMENTUM] = (int32_t)nmom;
    info->blocks[MUON_KIND_GRAM] = (int32_t)concat_tables(t, kGram).size();
    info->blocks[MUON_KIND_POLY] = (int32_t)concat_tables(t, kPoly).size();
    info->blocks[MUON_KIND_UPDATE] = (int32_t)concat_tables(t, kUpd).size();
    info->blocks[MUON_KIND_APPLY] = info->blocks[MUON_KIND_MOMENTUM];
    info->blocks[MUON_KIND_NORM] = n;
    info->x_master_iters = o.kmaster;
    info->path = o.path;
    int nf = 0;
    for (const Geometry& g : geo) nf += g.f32;
    info->n_f32_matrices = nf;
    int ng = 0;
    for (int grp = 0; grp < kGroups; ++grp) ng += !t.mom[grp].empty();
    info->n_groups = ng;
    info->fused = o.fused;
    info->blocks[MUON_KIND_FUSED] = (int32_t)t.fq.size();
  }
  if (kind == MUON_KIND_FUSED) {
    if (n_tiles) *n_tiles = (int32_t)t.fq.size();
    if (tiles) {
      const int cnt = std::min<int>(tile_cap, (int)t.fq.size());
      for (int x = 0; x < kXcds; ++x)
        for (int q = t.qoff[x]; q < t.qoff[x] + t.qlen[x] && q < cnt; ++q) {
          const Tile& tl = t.fq[q];
          int32_t* o5 = tiles + 5 * q;
          o5[0] = x;
          o5[1] = tl.pad;
          o5[2] = tl.mat;
          o5[3] = tl.ti;
          o5[4] = tl.tj;
        }
    }
  } else if (kind >= 0) {
    std::vector<Tile> v;
    switch (kind) {
      case MUON_KIND_MOMENTUM:
      case MUON_KIND_APPLY:
        for (int grp = 0; grp < kGroups; ++grp) v.insert(v.end(), t.mom[grp].begin(), t.mom[grp].end());
        break;
      case MUON_KIND_GRAM:
      case MUON_KIND_POLY:
      case MUON_KIND_UPDATE: {
        const int k = kind == MUON_KIND_GRAM ? kGram : kind == MUON_KIND_POLY ? kPoly : kUpd;
        v = concat_tables(t, k);
        break;
      }
      default: return fail(MUON_E_INVAL, "kind %d unknown", kind);
    }
    if (n_tiles) *n_tiles = (int32_t)v.size();
    if (tiles) {
      const int cnt = std::min<int>(tile_cap, (int)v.size());
      for (int q = 0; q < cnt; ++q) {
        const Tile& tl = v[q];
        tiles[3 * q] = tl.mat == kNullMat ? -1 : tl.mat;
        tiles[3 * q + 1] = tl.ti;
        tiles[3 * q + 2] = tl.tj;
      }
    }
  }
  return MUON_OK;
}

int muon_init(const muon_matrix_desc* descs, int n, const muon_options* opts, void* workspace, size_t ws_bytes,
              void* hip_stream, muon_plan** out_plan) {
  g_err.clear();
  if (!out_plan) return fail(MUON_E_INVAL, "out_plan is NULL");
  *out_plan = nullptr;
  Options o;
  int rc = read_options(opts, &o);
  if (rc) return rc;
  rc = validate_all(descs, n, true);
  if (rc) return rc;
  if (!workspace) return fail(MUON_E_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)workspace % kAlign) return fail(MUON_E_WORKSPACE, "workspace is not 256-byte aligned");

  muon_plan* p = new (std::nothrow) muon_plan();
  if (!p) return fail(MUON_E_INVAL, "out of host memory");
  p->n = n;
  p->opt = o;
  p->desc.assign(descs, descs + n);
  p->geo.resize(n);
  for (int i = 0; i < n; ++i) p->geo[i] = geometry(descs[i], o.path);
  p->tab = build_tables(p->geo, o.groups, o.fused);
  const size_t need = layout(p->geo, o, p->tab, &p->lay);
  if (ws_bytes < need) {
    delete p;
    return fail(MUON_E_WORKSPACE, "workspace has %zu bytes, the plan needs %zu", ws_bytes, need);
  }
  p->ws = (char*)workspace;
  p->ws_bytes = ws_bytes;
  hipStream_t stream = (hipStream_t)hip_stream;

  auto cleanup = [&](int code) {
    release(p);
    return code;
  };
  for (int s = 0; s < kSlots; ++s) {
    hipError_t e = hipHostMalloc((void**)&p->host_slots[s], sizeof(DevMat) * n, hipHostMallocDefault);
    if (e != hipSuccess) return cleanup(hip_fail(e, "hipHostMalloc(table staging)"));
    e = hipEventCreateWithFlags(&p->slot_ev[s], hipEventDisableTiming);
    if (e != hipSuccess) return cleanup(hip_fail(e, "hipEventCreate"));
  }
  hipError_t e = hipEventCreateWithFlags(&p->last_ev, hipEventDisableTiming);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipEventCreate"));
  e = hipEventCreateWithFlags(&p->fork_ev, hipEventDisableTiming);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipEventCreate"));
  for (int g = 0; g < kGroups; ++g) {
    e = hipStreamCreateWithFlags(&p->gs[g], hipStreamNonBlocking);
    if (e != hipSuccess) return cleanup(hip_fail(e, "hipStreamCreate"));
    e = hipEventCreateWithFlags(&p->join_ev[g], hipEventDisableTiming);
    if (e != hipSuccess) return cleanup(hip_fail(e, "hipEventCreate"));
  }
  e = prepare_stage_kernels();
  if (e == hipSuccess) e = prepare_bf16_kernels();
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipFuncSetAttribute(dynamic LDS)"));

  // Tile tables: staged through pinned memory, uploaded once; init waits for
  // them so the staging can be released.
  std::vector<std::pair<const std::vector<Tile>*, size_t>> lists;
  for (int grp = 0; grp < kGroups; ++grp) lists.push_back({&p->tab.mom[grp], p->lay.mom_tiles[grp]});
  for (int grp = 0; grp < kGroups; ++grp)
    for (int prec = 0; prec < 2; ++prec)
      for (int k = 0; k < 3; ++k) lists.push_back({&p->tab.ns[grp][prec][k], p->lay.ns_tiles[grp][prec][k]});
  lists.push_back({&p->tab.fq, p->lay.fq});
  size_t tb = 0;
  for (auto& l : lists) tb += sizeof(Tile) * l.first->size();
  void* stage = nullptr;
  e = hipHostMalloc(&stage, std::max<size_t>(tb, 16), hipHostMallocDefault);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipHostMalloc(tile staging)"));
  char* sp = (char*)stage;
  for (auto& l : lists) {
    const size_t bytes = sizeof(Tile) * l.first->size();
    if (!bytes) continue;
    std::memcpy(sp, l.first->data(), bytes);
    e = hipMemcpyAsync(p->ws + l.second, sp, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) {
      (void)hipHostFree(stage);
      return cleanup(hip_fail(e, "hipMemcpyAsync(tile tables)"));
    }
    sp += bytes;
  }
  p->hmat.resize(n);
  for (int i = 0; i < n; ++i) p->hmat[i] = make_devmat(p, i);
  p->slot = kSlots - 1;
  rc = upload_table(p, stream);
  if (rc) {
    (void)hipHostFree(stage);
    return cleanup(rc);
  }
  if (!p->tab.fq.empty()) {  // claim counters and the status word (the norm launch resets the counters)
    e = hipMemsetAsync(p->ws + p->lay.fctl, 0, sizeof(int32_t) * (kXcds + 1), stream);
    if (e != hipSuccess) {
      (void)hipHostFree(stage);
      return cleanup(hip_fail(e, "hipMemsetAsync(fused counters)"));
    }
  }
  if (o.zero) {
    for (int i = 0; i < n; ++i) {
      e = hipMemsetAsync(descs[i].momentum, 0, sizeof(float) * descs[i].rows * descs[i].cols, stream);
      if (e != hipSuccess) {
        (void)hipHostFree(stage);
        return cleanup(hip_fail(e, "hipMemsetAsync(momentum)"));
      }
    }
  }
  e = hipStreamSynchronize(stream);
  (void)hipHostFree(stage);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipStreamSynchronize(init upload)"));
  *out_plan = p;
  return MUON_OK;
}

// One step; iteration t uses sched[3(t-1) .. 3(t-1)+2] when sched is given, else (a, b, c).
static int enqueue_step(muon_plan* p, const DevMat* mats, const float* sched, float a, float b, float c, int T,
                        float momentum, int nesterov, float lr, hipStream_t stream);

static int step_impl(muon_plan* p, const muon_matrix_desc* descs, int n, const float* sched, float a, float b,
                     float c, int T, float momentum, int nesterov, float lr, void* hip_stream) {
  g_err.clear();
  if (!p) return fail(MUON_E_INVAL, "plan is NULL");
  if (T < 0 || T > p->opt.maxT) return fail(MUON_E_INVAL, "T=%d outside [0, max_T=%d]", T, p->opt.maxT);
  if (sched) {
    for (int q = 0; q < 3 * T; ++q)
      if (!std::isfinite(sched[q])) return fail(MUON_E_INVAL, "schedule entry %d (iteration %d) is not finite", q, q / 3 + 1);
  } else if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) {
    return fail(MUON_E_INVAL, "a, b and c must be finite");
  }
  if (!std::isfinite(lr)) return fail(MUON_E_INVAL, "lr must be finite");
  if (!(momentum >= 0.f && momentum <= 1.f)) return fail(MUON_E_INVAL, "momentum %g outside [0, 1]", momentum);
  hipStream_t stream = (hipStream_t)hip_stream;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t ce = hipStreamIsCapturing(stream, &cap);
  if (ce != hipSuccess) return hip_fail(ce, "hipStreamIsCapturing");
  const bool capturing = cap != hipStreamCaptureStatusNone;
  if (capturing && p->prof) return fail(MUON_E_INVAL, "profiling is on: a timed step cannot be captured in a graph");

  bool changed = false;
  if (descs) {
    if (n != p->n) return fail(MUON_E_MISMATCH, "step has %d matrices, the plan %d", n, p->n);
    int rc = validate_all(descs, n, true);
    if (rc) return rc;
    for (int i = 0; i < n; ++i) {
      const muon_matrix_desc& x = descs[i];
      const muon_matrix_desc& y = p->desc[i];
      if (x.rows != y.rows || x.cols != y.cols || x.g_dtype != y.g_dtype || x.w_dtype != y.w_dtype ||
          x.scale != y.scale)
        return fail(MUON_E_MISMATCH, "matrix %d: shape, dtype or scale differs from the plan", i);
      if (x.weight != y.weight || x.grad != y.grad || x.momentum != y.momentum) changed = true;
    }
    if (changed && (capturing || p->captured))
      return fail(MUON_E_INVAL,
                  "matrix pointers changed %s: a captured step reads the plan's matrix table, which a pointer "
                  "change rewrites; use a new plan for new buffers",
                  capturing ? "while the stream is capturing a graph" : "after a step of this plan was captured");
    if (changed) {
      for (int i = 0; i < n; ++i) {
        p->desc[i].weight = descs[i].weight;
        p->desc[i].grad = descs[i].grad;
        p->desc[i].momentum = descs[i].momentum;
        p->hmat[i] = make_devmat(p, i);
      }
      int rc2 = upload_table(p, stream);
      if (rc2) return rc2;
    }
  }

  int rc = enqueue_step(p, slot_ptr(p, p->slot), sched, a, b, c, T, momentum, nesterov, lr, stream);
  if (rc) return rc;
  if (capturing) p->captured = true;
  return note_slot_use(p, stream);
}

// Enqueue one step's launches over the plan's matrices (table `mats`, already
// on the device) on `stream`.
static int enqueue_step(muon_plan* p, const DevMat* mats, const float* sched, float a, float b, float c, int T,
                        float momentum, int nesterov, float lr, hipStream_t stream) {
  static const int kKinds[3] = {MUON_KIND_GRAM, MUON_KIND_POLY, MUON_KIND_UPDATE};
  static const char* kNames[3] = {"gram launch", "poly launch", "update launch"};
  LaunchEvents ev;
  int rc;

  // Each group's whole step (momentum, norm, T iterations) runs on a stream of
  // its own: the first on the caller's stream, the others forked from it and
  // joined back into it.  Starting group 1's momentum pass only after group
  // 0's measured slower.
  // fused plans run every bf16 product of a step in one launch when the
  // step's coefficients fit its arguments
  const bool fuse = !p->tab.fq.empty() && T >= 1 && T <= kFusedMaxT;
  bool busy[kGroups];
  int ngroups = 0;
  for (int grp = 0; grp < kGroups; ++grp) {
    busy[grp] = !p->tab.mom[grp].empty();
    ngroups += busy[grp];
  }
  // The first busy group runs on the caller's stream itself: between two
  // steps it then waits for one event hop (the other groups' joins) instead of
  // three (joins, fork record, fork wait); measured 1.87 against 1.90 ms.
  const bool fork = ngroups > 1;
  int home = 0;
  while (home < kGroups && !busy[home]) ++home;
  auto group_stream = [&](int grp) { return !fork || grp == home ? stream : p->gs[grp]; };
  hipError_t e = hipSuccess;
  if (fork) {
    e = hipEventRecord(p->fork_ev, stream);
    for (int grp = 0; grp < kGroups && e == hipSuccess; ++grp)
      if (busy[grp] && grp != home) e = hipStreamWaitEvent(p->gs[grp], p->fork_ev, 0);
    if (e != hipSuccess) return hip_fail(e, "fork of the group streams");
  }
  // Launch phase 0 is momentum plus norm (or apply when T = 0); phase
  // 3 (t - 1) + k + 1 is product k of iteration t.  The groups' launches are
  // enqueued phase by phase, alternating between the groups, so that every
  // group stream has work queued early even when the host enqueues slower
  // than the GPU runs.
  auto enqueue = [&](int grp, int phase) -> int {
    hipStream_t s = group_stream(grp);
    if (phase == 0) {
      const Tile* mom_tiles = (const Tile*)(p->ws + p->lay.mom_tiles[grp]);
      const int nmom = (int)p->tab.mom[grp].size();
      MomArgs ma{mats, mom_tiles, momentum, nesterov ? 1 : 0};
      if ((rc = prof_events(p, MUON_KIND_MOMENTUM, &ev))) return rc;
      if ((rc = check_launch(launch_momentum(ma, nmom, s, ev.start, ev.stop), "momentum launch"))) return rc;
      if (T == 0) {
        ApplyArgs aa{mats, mom_tiles, lr};
        if ((rc = prof_events(p, MUON_KIND_APPLY, &ev))) return rc;
        if ((rc = check_launch(launch_apply(aa, nmom, s, ev.start, ev.stop), "apply launch"))) return rc;
      } else {
        const int f0 = p->tab.first[grp], nf = p->tab.first[grp + 1] - f0;
        if ((rc = prof_events(p, MUON_KIND_NORM, &ev))) return rc;
        if ((rc = check_launch(launch_norm(mats + f0, nf, s, ev.start, ev.stop), "norm launch"))) return rc;
      }
      return MUON_OK;
    }
    const int t = (phase - 1) / 3 + 1, k = (phase - 1) % 3;
    if (fuse && phase == 1) {  // every bf16 product of the step, then the fp32 ones (if any) by launch
      FusedArgs fa;
      std::memset(&fa, 0, sizeof(fa));
      fa.mats = mats;
      fa.queue = (const Tile*)(p->ws + p->lay.fq);
      for (int x = 0; x < kXcds; ++x) {
        fa.qoff[x] = p->tab.qoff[x];
        fa.qlen[x] = p->tab.qlen[x];
      }
      fa.heads = (int32_t*)(p->ws + p->lay.fctl);
      fa.status = fa.heads + kXcds;
      fa.T = T;
      fa.kmaster = p->opt.kmaster;
      for (int q = 0; q < T; ++q) {
        fa.coef[q][0] = sched ? sched[3 * q] : a;
        fa.coef[q][1] = sched ? sched[3 * q + 1] : b;
        fa.coef[q][2] = sched ? sched[3 * q + 2] : c;
      }
      fa.lr = lr;
      fa.spin_limit = p->spin_limit;
      fa.dep_bias = p->dep_bias;
      if ((rc = prof_events(p, MUON_KIND_FUSED, &ev))) return rc;
      if ((rc = check_launch(launch_fused(fa, kProductGrid, s, ev.start, ev.stop), "fused launch"))) return rc;
    }
    for (int prec = fuse ? 1 : 0; prec < 2; ++prec) {
      const int ntab = (int)p->tab.ns[grp][prec][k].size();
      if (!ntab) continue;
      const float* tc = sched ? sched + 3 * (t - 1) : nullptr;
      StageArgs sa{mats, (const Tile*)(p->ws + p->lay.ns_tiles[grp][prec][k]), ntab, t, T, p->opt.kmaster,
                   tc ? tc[0] : a, tc ? tc[1] : b, tc ? tc[2] : c, lr};
      // the stride the table was laid out for, or fewer blocks when the
      // table is shorter (a multiple of 8: every block keeps its XCD)
      const int grid = std::min((ntab + 7) / 8 * 8, kProductGrid);
      if ((rc = prof_events(p, kKinds[k], &ev))) return rc;
      const hipError_t le = prec == 1 ? launch_stage(k + 1, true, sa, grid, s, ev.start, ev.stop)
                                      : launch_stage_bf16(k + 1, sa, grid, s, ev.start, ev.stop);
      if ((rc = check_launch(le, kNames[k]))) return rc;
    }
    return MUON_OK;
  };
  for (int phase = 0; phase <= 3 * T; ++phase)
    for (int grp = 0; grp < kGroups; ++grp)
      if (busy[grp] && (rc = enqueue(grp, phase))) return rc;
  if (fork) {
    for (int grp = 0; grp < kGroups; ++grp) {
      if (!busy[grp] || grp == home) continue;
      e = hipEventRecord(p->join_ev[grp], p->gs[grp]);
      if (e == hipSuccess) e = hipStreamWaitEvent(stream, p->join_ev[grp], 0);
      if (e != hipSuccess) return hip_fail(e, "join of the group streams");
    }
  }
  return MUON_OK;
}

int muon_step(muon_plan* p, const muon_matrix_desc* descs, int n, float a, float b, float c, int T, float momentum,
              int nesterov, float lr, void* hip_stream) {
  return step_impl(p, descs, n, nullptr, a, b, c, T, momentum, nesterov, lr, hip_stream);
}

int muon_step_schedule(muon_plan* p, const muon_matrix_desc* descs, int n, const float* coeffs, int T,
                       float momentum, int nesterov, float lr, void* hip_stream) {
  if (!coeffs && T > 0) {
    g_err.clear();
    return fail(MUON_E_INVAL, "coeffs is NULL with T=%d", T);
  }
  return step_impl(p, descs, n, coeffs, 0.f, 0.f, 0.f, T, momentum, nesterov, lr, hip_stream);
}

namespace {
// Frees a plan's host state; leaves the thread's error message alone (init's
// failure paths call it after recording what failed).
void release(muon_plan* p) {
  if (!p) return;
  if (p->last_valid) (void)hipEventSynchronize(p->last_ev);
  for (int s = 0; s < kSlots; ++s) {
    if (p->host_slots[s]) (void)hipHostFree(p->host_slots[s]);
    if (p->slot_ev[s]) (void)hipEventDestroy(p->slot_ev[s]);
  }
  if (p->last_ev) (void)hipEventDestroy(p->last_ev);
  if (p->fork_ev) (void)hipEventDestroy(p->fork_ev);
  for (int g = 0; g < kGroups; ++g) {
    if (p->join_ev[g]) (void)hipEventDestroy(p->join_ev[g]);
    if (p->gs[g]) (void)hipStreamDestroy(p->gs[g]);
  }
  for (hipEvent_t ev : p->pev) (void)hipEventDestroy(ev);
  delete p;
}
}  // namespace

int muon_destroy(muon_plan* p) {
  g_err.clear();
  release(p);
  return MUON_OK;
}

int muon_profile_enable(muon_plan* p, int enable) {
  g_err.clear();
  if (!p) return fail(MUON_E_INVAL, "plan is NULL");
  p->prof = enable != 0;
  return MUON_OK;
}

int muon_profile_select(muon_plan* p, uint32_t kind_mask) {
  g_err.clear();
  if (!p) return fail(MUON_E_INVAL, "plan is NULL");
  p->pmask = kind_mask;
  return MUON_OK;
}

int muon_check(muon_plan* p, void* hip_stream) {
  g_err.clear();
  if (!p) return fail(MUON_E_INVAL, "plan is NULL");
  if (p->tab.fq.empty()) return MUON_OK;
  hipStream_t stream = (hipStream_t)hip_stream;
  int32_t* status = (int32_t*)(p->ws + p->lay.fctl) + kXcds;
  int32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, status, sizeof(h), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "muon_check: reading the fused launch status");
  if (h == 0) return MUON_OK;
  e = hipMemsetAsync(status, 0, sizeof(int32_t), stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "muon_check: clearing the fused launch status");
  if (h & kFusedBadEntry)
    return fail(MUON_E_HIP, "fused launch: a queue entry lies outside its matrix (status %d); the blocks stopped "
                "and that step's results are incomplete", (int)h);
  return fail(MUON_E_HIP,
              "fused launch: a dependency wait gave up after %d polls (status %d); the blocks stopped and that "
              "step's results are incomplete",
              p->spin_limit, (int)h);
}

int muon_fused_limits(muon_plan* p, int32_t spin_limit, int32_t dep_bias) {
  g_err.clear();
  if (!p) return fail(MUON_E_INVAL, "plan is NULL");
  if (p->tab.fq.empty()) return fail(MUON_E_INVAL, "the plan is not fused");
  if (spin_limit <= 0 || dep_bias < 0) return fail(MUON_E_INVAL, "spin_limit %d must be > 0, dep_bias %d >= 0", spin_limit, dep_bias);
  p->spin_limit = spin_limit;
  p->dep_bias = dep_bias;
  return MUON_OK;
}

int muon_profile_read(muon_plan* p, double* ms, int64_t* launches) {
  g_err.clear();
  if (!p) return fail(MUON_E_INVAL, "plan is NULL");
  for (size_t q = 0; q < p->pused; ++q) {
    hipError_t e = hipEventSynchronize(p->pev[2 * q + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(profile)");
    float t = 0.f;
    e = hipEventElapsedTime(&t, p->pev[2 * q], p->pev[2 * q + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    p->pms[p->pkind[q]] += t;
    p->pcnt[p->pkind[q]] += 1;
  }
  p->pused = 0;
  for (int k = 0; k < MUON_KIND_COUNT; ++k) {
    if (ms) ms[k] = p->pms[k];
    if (launches) launches[k] = p->pcnt[k];
    p->pms[k] = 0.0;
    p->pcnt[k] = 0;
  }
  return MUON_OK;
}

}  // extern "C"

// ---------------------------------------------------- allocation-free step --
//
// The step's working memory (X copies, A, B, partial sums, tables) lives in
// this file-scope array instead of a caller workspace.  Every GPU the library
// runs on holds its own copy, from module load to the end of the process.
// Host code never passes the array's name to a kernel or a copy: it passes
// the device address taken once per device with hipGetSymbolAddress.
namespace {
constexpr size_t kScratchBytes = MUON_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};      // device address of `scratch`, per device
std::vector<char> g_scratch_host[kMaxDevices];  // pageable staging of the tables, per device
hipEvent_t g_scratch_ev[kMaxDevices] = {};  // recorded after the last table copy out of that staging
bool g_scratch_ev_used[kMaxDevices] = {};

// Device address of the current device's scratch array (taken on the first
// call on that device, with the device current), its host staging buffer and
// the event that guards the buffer's reuse.
int scratch_for_current_device(void** dev_ptr, std::vector<char>** host, int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || (uintptr_t)ptr % kAlign) return fail(MUON_E_HIP, "scratch array address %p is not 256-byte aligned", ptr);
    e = prepare_stage_kernels();
    if (e == hipSuccess) e = prepare_bf16_kernels();
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute(dynamic LDS)");
    e = hipEventCreateWithFlags(&g_scratch_ev[dev], hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate(scratch tables)");
    g_scratch_dev[dev] = ptr;
  }
  *dev_ptr = g_scratch_dev[dev];
  *host = &g_scratch_host[dev];
  *dev_out = dev;
  return MUON_OK;
}
}  // namespace

int muon_step_scratch(const muon_matrix_desc* descs, int n, const muon_options* opts, float a, float b, float c,
                      int T, float momentum, int nesterov, float lr, void* hip_stream) {
  g_err.clear();
  Options o;
  int rc = read_options(opts, &o);
  if (rc) return rc;
  if (o.zero) return fail(MUON_E_INVAL, "options.zero_momentum is not supported by muon_step_scratch");
  o.groups = 1;  // one stream: the caller's
  o.fused = 0;   // the three launches per iteration: a fused launch keeps per-plan counters
  if (T < 0 || T > o.maxT) return fail(MUON_E_INVAL, "T=%d outside [0, max_T=%d]", T, o.maxT);
  if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) return fail(MUON_E_INVAL, "a, b and c must be finite");
  if (!std::isfinite(lr)) return fail(MUON_E_INVAL, "lr must be finite");
  if (!(momentum >= 0.f && momentum <= 1.f)) return fail(MUON_E_INVAL, "momentum %g outside [0, 1]", momentum);
  rc = validate_all(descs, n, true);
  if (rc) return rc;

  muon_plan p;  // host state of this call only: no streams, events or pinned memory
  p.n = n;
  p.opt = o;
  p.desc.assign(descs, descs + n);
  p.geo.resize(n);
  for (int i = 0; i < n; ++i) p.geo[i] = geometry(descs[i], o.path);
  p.tab = build_tables(p.geo, o.groups, false);
  const size_t need = layout(p.geo, o, p.tab, &p.lay);
  if (need > kScratchBytes)
    return fail(MUON_E_WORKSPACE, "this step needs %zu bytes of scratch; muon_step_scratch holds %zu (use muon_init "
                "with a workspace)", need, kScratchBytes);
  void* dev_scratch = nullptr;
  std::vector<char>* host = nullptr;
  int dev = 0;
  rc = scratch_for_current_device(&dev_scratch, &host, &dev);
  if (rc) return rc;
  // the previous call's table copies must have read the staging buffer
  if (g_scratch_ev_used[dev]) {
    hipError_t e = hipEventSynchronize(g_scratch_ev[dev]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(scratch tables)");
  }
  p.ws = (char*)dev_scratch;
  p.ws_bytes = kScratchBytes;
  p.hmat.resize(n);
  for (int i = 0; i < n; ++i) p.hmat[i] = make_devmat(&p, i);

  // Tile tables and the matrix table, staged in this device's pageable host
  // buffer and copied into the scratch array on the caller's stream.
  hipStream_t stream = (hipStream_t)hip_stream;
  std::vector<std::pair<const void*, std::pair<size_t, size_t>>> parts;  // (source, (scratch offset, bytes))
  for (int grp = 0; grp < kGroups; ++grp)
    parts.push_back({p.tab.mom[grp].data(), {p.lay.mom_tiles[grp], sizeof(Tile) * p.tab.mom[grp].size()}});
  for (int grp = 0; grp < kGroups; ++grp)
    for (int prec = 0; prec < 2; ++prec)
      for (int k = 0; k < 3; ++k)
        parts.push_back({p.tab.ns[grp][prec][k].data(),
                         {p.lay.ns_tiles[grp][prec][k], sizeof(Tile) * p.tab.ns[grp][prec][k].size()}});
  parts.push_back({p.hmat.data(), {p.lay.slots, sizeof(DevMat) * n}});
  size_t total = 0;
  for (auto& q : parts) total += q.second.second;
  host->resize(std::max<size_t>(total, 16));
  char* hp = host->data();
  for (auto& q : parts) {
    const size_t bytes = q.second.second;
    if (!bytes) continue;
    std::memcpy(hp, q.first, bytes);
    hipError_t e = hipMemcpyAsync(p.ws + q.second.first, hp, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(tables into scratch)");
    hp += bytes;
  }
  hipError_t e = hipEventRecord(g_scratch_ev[dev], stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(scratch tables)");
  g_scratch_ev_used[dev] = true;
  return enqueue_step(&p, (const DevMat*)(p.ws + p.lay.slots), nullptr, a, b, c, T, momentum, nesterov, lr, stream);
}
