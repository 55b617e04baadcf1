// gfx950 (CDNA4) kernels of the Muon step.
//
// The method (guide page "NanoGPT Speedrun: The Ultimate Guide ...", section
// "Optimizer and Training Strategy Tuning"; overview page "The NanoGPT
// speedrun", paragraph "Six records account for most of the speedup"):
// Nesterov momentum, then replace the update by its nearest semi-orthogonal
// matrix via Newton-Schulz steps, then apply it to the weights.
//
//   momentum_kernel   M <- mu M + G (one fp32 rounding), U = G + mu M or M,
//                     per-tile partial sums of U^2, X0 = U written in the
//                     canonical (short side first) orientation, fp32 and/or bf16.
//   ns_stage_kernel<1> A = s^2 X X^T     (upper tiles, mirrored store)
//   ns_stage_kernel<2> B = b A + c A A    (A symmetric: A A = A A^T)
//   ns_stage_kernel<3> X <- a X + B X; on the last step W <- W - lr s O
//   apply_kernel       T == 0: W <- W - lr s X0
//
// The three products share one MFMA main loop: 128x128 output tile per
// 256-thread block, 4 waves each owning 64x64 as 2x2 v_mfma_f32_32x32x16_bf16
// (or v_mfma_f32_32x32x2_f32 on the fp32 path), K staged through LDS in
// 128-byte rows with an XOR swizzle, double-buffered through registers.
#include <hip/hip_runtime.h>

#include "muon_internal.h"

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers --

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  u32x2 r;
  r.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
  r.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
  return r;
}
__device__ __forceinline__ void unpack4_bf16(u32x2 r, float* v) {
  v[0] = __uint_as_float(r.x << 16);
  v[1] = __uint_as_float(r.x & 0xFFFF0000u);
  v[2] = __uint_as_float(r.y << 16);
  v[3] = __uint_as_float(r.y & 0xFFFF0000u);
}

// LDS row swizzle: 16-byte chunk c of tile row r lives at chunk c ^ swz(r).
// Any 8 consecutive rows get 8 distinct chunks (conflict-free fragment reads),
// and rows 8 apart differ too (conflict-light transposed writes).
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 1 / (||U||_F + eps) from the momentum kernel's partial sums, summed in a
// fixed order (deterministic); every thread of the block gets the result.
// `scratch` needs 256 doubles of shared memory.
__device__ __forceinline__ float block_inv_norm(const DevMat& d, double* scratch, double* nu_out) {
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int p = tid; p < d.nparts; p += kThreads) s += (double)d.part[p];
  scratch[tid] = s;
  __syncthreads();
#pragma unroll
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) scratch[tid] += scratch[tid + w];
    __syncthreads();
  }
  const double nu = sqrt(scratch[0]);
  __syncthreads();  // scratch may be reused right after
  if (nu_out) *nu_out = nu;
  return (float)(1.0 / (nu + kEps));
}

// ---------------------------------------------------------- momentum ------

// One 64x64 tile of the canonical X per block.  Thread (tx, ty) handles 4
// consecutive columns of rows ty, ty+16, ty+32, ty+48 of the ORIGINAL tile,
// so gradient and momentum accesses are coalesced along the original rows.
__global__ __launch_bounds__(kThreads) void momentum_kernel(MomArgs args) {
  const Tile tl = args.tiles[blockIdx.x];
  if (tl.mat == kNullMat) return;
  const DevMat& d = args.mats[tl.mat];
  __shared__ float stage[kMomTile][kMomTile + 1];
  __shared__ float red[kThreads / 64];

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int i0 = tl.ti * kMomTile, j0 = tl.tj * kMomTile;  // canonical origin
  const bool tr = d.transposed != 0;
  const int r0 = tr ? j0 : i0, c0 = tr ? i0 : j0;          // original origin
  const float mu = args.mu;

  float u[4][4];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + ty + 16 * q;
    const int c = c0 + 4 * tx;
    float g[4] = {0.f, 0.f, 0.f, 0.f}, m[4] = {0.f, 0.f, 0.f, 0.f};
    bool ok[4];
    const bool rowok = r < d.rows;
    const size_t off = (size_t)r * d.cols + c;
    if (rowok && d.vec_g && c + 3 < d.cols) {
      if (d.g_bf16) {
        unpack4_bf16(*(const u32x2*)((const uint16_t*)d.g + off), g);
      } else {
        f32x4 gv = *(const f32x4*)((const float*)d.g + off);
        g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
      }
      f32x4 mv = *(const f32x4*)(d.mom + off);
      m[0] = mv.x; m[1] = mv.y; m[2] = mv.z; m[3] = mv.w;
#pragma unroll
      for (int e = 0; e < 4; ++e) ok[e] = true;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ok[e] = rowok && (c + e) < d.cols;
        if (ok[e]) {
          g[e] = d.g_bf16 ? bf2f(((const uint16_t*)d.g)[off + e]) : ((const float*)d.g)[off + e];
          m[e] = d.mom[off + e];
        }
      }
    }
    float mn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn[e] = fmaf(mu, m[e], g[e]);  // one rounding: fl32(mu*M + G)
      const float ue = args.nesterov ? fmaf(mu, mn[e], g[e]) : mn[e];
      u[q][e] = ok[e] ? ue : 0.f;
      ss = fmaf(u[q][e], u[q][e], ss);
    }
    if (rowok && d.vec_g && c + 3 < d.cols) {
      *(f32x4*)(d.mom + off) = f32x4{mn[0], mn[1], mn[2], mn[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok[e]) d.mom[off + e] = mn[e];
    }
  }

  // X0 = U in the canonical orientation (zero in the padding).
  float xv[4][4];
  if (tr) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) stage[ty + 16 * q][4 * tx + e] = u[q][e];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[q][e] = stage[4 * tx + e][ty + 16 * q];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[q][e] = u[q][e];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const size_t xo = (size_t)(i0 + ty + 16 * q) * d.np + j0 + 4 * tx;
    if (d.f32) {
      *(f32x4*)((float*)d.xo[0] + xo) = f32x4{xv[q][0], xv[q][1], xv[q][2], xv[q][3]};
    } else {
      *(u32x2*)((uint16_t*)d.xo[0] + xo) = pack4_bf16(xv[q][0], xv[q][1], xv[q][2], xv[q][3]);
      if (d.x32) *(f32x4*)(d.x32 + xo) = f32x4{xv[q][0], xv[q][1], xv[q][2], xv[q][3]};
    }
  }

  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) d.part[tl.ti * d.mom_tiles_n + tl.tj] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ------------------------------------------------------ weight step -------

template <bool W_BF16>
__device__ __forceinline__ void weight_step4(const DevMat& d, int i, int j, const float* o, float lr_eff) {
  // canonical (i, j..j+3) -> original (i, j+e) or (j+e, i)
  if (i >= d.m) return;
  if (!d.transposed) {
    const size_t off = (size_t)i * d.cols + j;
    if (d.vec_w && j + 3 < d.n) {
      if (W_BF16) {
        u32x2* p = (u32x2*)((uint16_t*)d.w + off);
        float w[4];
        unpack4_bf16(*p, w);
        *p = pack4_bf16(fmaf(-lr_eff, o[0], w[0]), fmaf(-lr_eff, o[1], w[1]),
                        fmaf(-lr_eff, o[2], w[2]), fmaf(-lr_eff, o[3], w[3]));
      } else {
        f32x4* p = (f32x4*)((float*)d.w + off);
        f32x4 w = *p;
        w.x = fmaf(-lr_eff, o[0], w.x);
        w.y = fmaf(-lr_eff, o[1], w.y);
        w.z = fmaf(-lr_eff, o[2], w.z);
        w.w = fmaf(-lr_eff, o[3], w.w);
        *p = w;
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j + e >= d.n) break;
      if (W_BF16) {
        uint16_t* p = (uint16_t*)d.w + off + e;
        *p = f2bf(fmaf(-lr_eff, o[e], bf2f(*p)));
      } else {
        float* p = (float*)d.w + off + e;
        *p = fmaf(-lr_eff, o[e], *p);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j + e >= d.n) break;
      const size_t off = (size_t)(j + e) * d.cols + i;
      if (W_BF16) {
        uint16_t* p = (uint16_t*)d.w + off;
        *p = f2bf(fmaf(-lr_eff, o[e], bf2f(*p)));
      } else {
        float* p = (float*)d.w + off;
        *p = fmaf(-lr_eff, o[e], *p);
      }
    }
  }
}

__device__ __forceinline__ void weight_step(const DevMat& d, int i, int j, const float* o, float lr_eff) {
  if (d.w_bf16)
    weight_step4<true>(d, i, j, o, lr_eff);
  else
    weight_step4<false>(d, i, j, o, lr_eff);
}

// T == 0: the update is X0 itself.  Same tiling as the momentum kernel.
__global__ __launch_bounds__(kThreads) void apply_kernel(ApplyArgs args) {
  const Tile tl = args.tiles[blockIdx.x];
  if (tl.mat == kNullMat) return;
  const DevMat& d = args.mats[tl.mat];
  __shared__ double scratch[kThreads];
  const float inv = block_inv_norm(d, scratch, nullptr);
  const float lr_eff = args.lr * d.scale * inv;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tl.ti * kMomTile + ty + 16 * q;
    const int j = tl.tj * kMomTile + 4 * tx;
    const size_t xo = (size_t)i * d.np + j;
    float u[4];
    if (d.f32) {
      f32x4 v = *(const f32x4*)((const float*)d.xo[0] + xo);
      u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
    } else if (d.x32) {
      f32x4 v = *(const f32x4*)(d.x32 + xo);
      u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
    } else {
      unpack4_bf16(*(const u32x2*)((const uint16_t*)d.xo[0] + xo), u);
    }
    weight_step(d, i, j, u, lr_eff);
  }
}

// ------------------------------------------------ Newton-Schulz stages ----

// Global -> register copy of a 128-row x 128-byte operand panel whose K runs
// along memory rows (row r of the panel = memory row row0 + r).
__device__ __forceinline__ void load_kc(u32x4 (&r)[4], const char* base, size_t ld_bytes, int kbyte0,
                                        int tid) {
  const int c = tid & 7, rr = tid >> 3;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = *(const u32x4*)(base + (size_t)(rr + 32 * q) * ld_bytes + kbyte0 + 16 * c);
}
__device__ __forceinline__ void store_kc(char* lds, const u32x4 (&r)[4], int tid) {
  const int c = tid & 7, rr = tid >> 3;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = rr + 32 * q;
    *(u32x4*)(lds + row * 128 + ((c ^ swz(row)) << 4)) = r[q];
  }
}

// Panel whose K runs down memory columns: element (j, k) of the panel is
// memory (k0 + k, j0 + j).  Each thread reads a 4(k) x 8(j) bf16 block (or
// 4 x 4 fp32) and writes it transposed, so LDS rows are again K-contiguous.
template <bool F32>
__device__ __forceinline__ void load_tr(u32x4 (&r)[4], const char* base, size_t ld_bytes, int k0, int jbyte0,
                                        int tid) {
  const int jg = F32 ? (tid & 31) : (tid & 15);
  const int kg = F32 ? (tid >> 5) : (tid >> 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = *(const u32x4*)(base + (size_t)(k0 + 4 * kg + q) * ld_bytes + jbyte0 + 16 * jg);
}
template <bool F32>
__device__ __forceinline__ void store_tr(char* lds, const u32x4 (&r)[4], int tid) {
  if (F32) {
    const int jg = tid & 31, kg = tid >> 5;  // kg = 16-byte chunk (4 floats of K)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * jg + e;
      *(u32x4*)(lds + row * 128 + ((kg ^ swz(row)) << 4)) = u32x4{r[0][e], r[1][e], r[2][e], r[3][e]};
    }
  } else {
    const int jg = tid & 15, kg = tid >> 4;  // 4 bf16 of K = half a chunk
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      const u32x2 ev{(r[0][dd] & 0xFFFFu) | (r[1][dd] << 16), (r[2][dd] & 0xFFFFu) | (r[3][dd] << 16)};
      const u32x2 od{(r[0][dd] >> 16) | (r[1][dd] & 0xFFFF0000u), (r[2][dd] >> 16) | (r[3][dd] & 0xFFFF0000u)};
      const int re = 8 * jg + 2 * dd, ro = re + 1;
      *(u32x2*)(lds + re * 128 + (((kg >> 1) ^ swz(re)) << 4) + ((kg & 1) << 3)) = ev;
      *(u32x2*)(lds + ro * 128 + (((kg >> 1) ^ swz(ro)) << 4) + ((kg & 1) << 3)) = od;
    }
  }
}

// acc[mi][nj] += P(j rows) x Q(i rows)^T over one 128-byte K slab in LDS.
// MFMA operand A = P fragment (MFMA row <-> output column j), operand B = Q
// fragment (MFMA column <-> output row i): each lane then holds 4
// consecutive output columns of one output row per 4 accumulator registers.
template <bool F32>
__device__ __forceinline__ void mma_slab(f32x16 (&acc)[2][2], const char* lq, const char* lp, int wm, int wn,
                                         int lane) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int chunk = 2 * ks + (lane >> 5);
    u32x4 qf[2], pf[2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int row = wm * 64 + mi * 32 + (lane & 31);
      qf[mi] = *(const u32x4*)(lq + row * 128 + ((chunk ^ swz(row)) << 4));
    }
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) {
      const int row = wn * 64 + nj * 32 + (lane & 31);
      pf[nj] = *(const u32x4*)(lp + row * 128 + ((chunk ^ swz(row)) << 4));
    }
    if (!F32) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pf[nj]),
                                                                 __builtin_bit_cast(bf16x8, qf[mi]),
                                                                 acc[mi][nj], 0, 0, 0);
    } else {
      // Four fp32 K values per lane: MFMA e takes element e; both operands use
      // the same K order, so the contraction covers all 32 K of the slab.
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int nj = 0; nj < 2; ++nj)
            acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(pf[nj][e]),
                                                                __uint_as_float(qf[mi][e]), acc[mi][nj], 0, 0, 0);
    }
  }
}

template <bool F32>
__device__ __forceinline__ void store4(void* base, size_t off, const float* v) {
  if (F32)
    *(f32x4*)((float*)base + off) = f32x4{v[0], v[1], v[2], v[3]};
  else
    *(u32x2*)((uint16_t*)base + off) = pack4_bf16(v[0], v[1], v[2], v[3]);
}
template <bool F32>
__device__ __forceinline__ void load4(const void* base, size_t off, float* v) {
  if (F32) {
    f32x4 x = *(const f32x4*)((const float*)base + off);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
    unpack4_bf16(*(const u32x2*)((const uint16_t*)base + off), v);
  }
}
template <bool F32>
__device__ __forceinline__ void store1(void* base, size_t off, float v) {
  if (F32)
    ((float*)base)[off] = v;
  else
    ((uint16_t*)base)[off] = f2bf(v);
}

// Symmetric store of a 4-column strip: row i, columns j..j+3 and the mirror.
// Diagonal tiles keep only i <= j' so both triangles hold the same values.
template <bool F32>
__device__ __forceinline__ void store_sym(void* out, int ld, int i, int j, const float* v, bool diag) {
  if (!diag) {
    store4<F32>(out, (size_t)i * ld + j, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) store1<F32>(out, (size_t)(j + e) * ld + i, v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i <= j + e) {
        store1<F32>(out, (size_t)i * ld + j + e, v[e]);
        store1<F32>(out, (size_t)(j + e) * ld + i, v[e]);
      }
  }
}

template <int STAGE, bool F32>
__global__ __launch_bounds__(kThreads, 2) void ns_stage_kernel(StageArgs args) {
  constexpr int ES = F32 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kTile * 128];

  const Tile tl = args.tiles[blockIdx.x];
  if (tl.mat == kNullMat) return;
  const DevMat& d = args.mats[tl.mat];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i0 = tl.ti * kTile, j0 = tl.tj * kTile;
  const int t = args.t;
  const char* xin = (const char*)d.xo[(t - 1) & 1];

  const char* qbase;
  const char* pbase;
  size_t q_ld, p_ld;
  int K;
  if (STAGE == 1) {
    q_ld = p_ld = (size_t)d.np * ES;
    qbase = xin + (size_t)i0 * q_ld;
    pbase = xin + (size_t)j0 * p_ld;
    K = d.np;
  } else if (STAGE == 2) {
    q_ld = p_ld = (size_t)d.mp * ES;
    qbase = (const char*)d.a + (size_t)i0 * q_ld;
    pbase = (const char*)d.a + (size_t)j0 * p_ld;
    K = d.mp;
  } else {
    q_ld = (size_t)d.mp * ES;
    qbase = (const char*)d.b + (size_t)i0 * q_ld;
    p_ld = (size_t)d.np * ES;
    pbase = xin;
    K = d.mp;
  }

  float pre = 1.f;  // stage 1 of the first iteration: A = s^2 U U^T
  if (STAGE == 1 && t == 1) {
    double nu;
    const float inv = block_inv_norm(d, (double*)smem, &nu);
    pre = inv * inv;
    if (tl.ti == 0 && tl.tj == 0 && tid == 0) {
      d.sc[0] = inv;
      d.sc[1] = (float)nu;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][nj][v] = 0.f;

  constexpr int BK = 128 / ES;  // K elements per 128-byte slab
  const int nk = K / BK;
  u32x4 rq[4], rp[4];
  load_kc(rq, qbase, q_ld, 0, tid);
  if (STAGE == 3)
    load_tr<F32>(rp, pbase, p_ld, 0, j0 * ES, tid);
  else
    load_kc(rp, pbase, p_ld, 0, tid);
  store_kc(smem, rq, tid);
  if (STAGE == 3)
    store_tr<F32>(smem + kTile * 128, rp, tid);
  else
    store_kc(smem + kTile * 128, rp, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_kc(rq, qbase, q_ld, (kt + 1) * 128, tid);
      if (STAGE == 3)
        load_tr<F32>(rp, pbase, p_ld, (kt + 1) * BK, j0 * ES, tid);
      else
        load_kc(rp, pbase, p_ld, (kt + 1) * 128, tid);
    }
    const char* lq = smem + buf * (2 * kTile * 128);
    mma_slab<F32>(acc, lq, lq + kTile * 128, wm, wn, lane);
    if (more) {
      char* nq = smem + (buf ^ 1) * (2 * kTile * 128);
      store_kc(nq, rq, tid);
      if (STAGE == 3)
        store_tr<F32>(nq + kTile * 128, rp, tid);
      else
        store_kc(nq + kTile * 128, rp, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds output row i, columns j..j+3 per 4 registers.
  const int h = lane >> 5;
  const bool diag = tl.ti == tl.tj;
  float alpha = args.a, beta = 1.f, lr_eff = 0.f;
  bool last = false, master32 = false, write32 = false;
  const void* xm = xin;
  if (STAGE == 3) {
    if (t == 1) {
      const float inv = d.sc[0];
      alpha = args.a * inv;
      beta = inv;
    }
    last = t == args.T;
    master32 = !F32 && t <= args.kmaster;
    write32 = !F32 && !last && t < args.kmaster;
    lr_eff = args.lr * d.scale;
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int i = i0 + wm * 64 + mi * 32 + (lane & 31);
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = j0 + wn * 64 + nj * 32 + 8 * g + 4 * h;
        float v[4] = {acc[mi][nj][4 * g], acc[mi][nj][4 * g + 1], acc[mi][nj][4 * g + 2], acc[mi][nj][4 * g + 3]};
        if (STAGE == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= pre;
          store_sym<F32>(d.a, d.mp, i, j, v, diag);
        } else if (STAGE == 2) {
          float av[4];
          load4<F32>(d.a, (size_t)i * d.mp + j, av);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(args.c, v[e], args.b * av[e]);
          store_sym<F32>(d.b, d.mp, i, j, v, diag);
        } else {
          const size_t off = (size_t)i * d.np + j;
          float xv[4];
          if (master32) {
            f32x4 x = *(const f32x4*)(d.x32 + off);
            xv[0] = x.x; xv[1] = x.y; xv[2] = x.z; xv[3] = x.w;
          } else {
            load4<F32>(xm, off, xv);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(alpha, xv[e], beta * v[e]);
          if (!last) {
            store4<F32>(d.xo[t & 1], off, v);
            if (write32) *(f32x4*)(d.x32 + off) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            weight_step(d, i, j, v, lr_eff);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------ launchers --

#define MUON_STAGE_LAUNCH(S, F)                                                              \
  hipLaunchKernelGGL((ns_stage_kernel<S, F>), dim3(blocks), dim3(kThreads), 0, stream, args); \
  break;

hipError_t launch_momentum(const MomArgs& args, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(momentum_kernel, dim3(blocks), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_apply(const ApplyArgs& args, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(apply_kernel, dim3(blocks), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_stage(int stage, bool f32, const StageArgs& args, int blocks, hipStream_t stream) {
  switch (stage * 2 + (f32 ? 1 : 0)) {
    case 2: MUON_STAGE_LAUNCH(1, false)
    case 3: MUON_STAGE_LAUNCH(1, true)
    case 4: MUON_STAGE_LAUNCH(2, false)
    case 5: MUON_STAGE_LAUNCH(2, true)
    case 6: MUON_STAGE_LAUNCH(3, false)
    case 7: MUON_STAGE_LAUNCH(3, true)
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
