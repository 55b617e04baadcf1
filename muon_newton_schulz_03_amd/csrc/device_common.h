// Device helpers shared by the gfx950 kernels of the Muon step: vector
// types, global-address-space views, bf16 packing, the (bf16, low byte)
// representation of X, buffer resources and wait/barrier forms, the
// transposing LDS fragment reads, and the persistent kernels' table walk.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <type_traits>

#include "muon_internal.h"

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Global-memory views of plain pointers.  The pointers in the matrix table are
// generic; accesses through these views compile to global_* instructions,
// which count only against the vector-memory counter (flat_* ones would also
// count against the LDS counter, so every LDS wait would wait for them).
#define MUON_GLOBAL __attribute__((address_space(1)))
template <class V, class T>
__device__ __forceinline__ MUON_GLOBAL V* gv(T* p) {
  return (MUON_GLOBAL V*)(void*)p;
}
template <class V, class T>
__device__ __forceinline__ const MUON_GLOBAL V* gv(const T* p) {
  return (const MUON_GLOBAL V*)(const void*)p;
}

// ---------------------------------------------------------------- helpers --

// A plain-typed copy of data the kernel only reads (table entries, a norm
// scale written by an earlier launch) through the constant address space:
// uniform addresses then compile to scalar loads, which do not share the
// in-order vector-memory counter with the epilogue's loads and stores.
#define MUON_CONST __attribute__((address_space(4)))
template <class T>
__device__ __forceinline__ T load_uniform(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "whole dwords");
  struct Words {
    uint32_t w[sizeof(T) / 4];
  } v;
  const MUON_CONST uint32_t* s = (const MUON_CONST uint32_t*)(const void*)p;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) v.w[i] = s[i];
  return __builtin_bit_cast(T, v);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// Low byte of the (hi, lo) pair that carries X in more precision than one
// bf16.  hi = bf16(x) is the operand copy itself.  In the integer order of
// fp32 bit patterns, x lies within 2^15 of hi (half of bf16's last place is
// 2^15 fp32 places); lo is that distance in units of 256, rounded to
// nearest, q = min((bits(x) - bits(hi) + 128) >> 8, 127), stored as a signed
// byte (the clamp only catches distances within 128 of 2^15).  The pair
// decodes to the fp32 pattern bits(hi) + 256 q: x to about 16 significant
// bits (relative error at most 2^-15, unbiased: rounding down in this order
// would shrink every |x|), in a few integer operations each way.
__device__ __forceinline__ uint32_t lo_byte(float x, uint32_t hi_bits) {
  const int r = (int)(__float_as_uint(x) - hi_bits);
  return (uint32_t)min((r + 128) >> 8, 127) & 0xFFu;
}
__device__ __forceinline__ float with_lo(uint32_t hi_bits, uint32_t lo_word, int e) {
  const int q = __builtin_amdgcn_sbfe((int)lo_word, 8 * e, 8);
  return __uint_as_float(hi_bits + ((uint32_t)q << 8));
}

// Two floats to two bf16 (RNE) in one word, low half first: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  return u32x2{pack2_bf16(a, b), pack2_bf16(c, d)};
}
__device__ __forceinline__ void unpack4_bf16(u32x2 r, float* v) {
  v[0] = __uint_as_float(r.x << 16);
  v[1] = __uint_as_float(r.x & 0xFFFF0000u);
  v[2] = __uint_as_float(r.y << 16);
  v[3] = __uint_as_float(r.y & 0xFFFF0000u);
}
// fp32 patterns of the 4 bf16 words packed by pack4_bf16.
__device__ __forceinline__ void hi_bits4(u32x2 hi, uint32_t* b) {
  b[0] = hi.x << 16;
  b[1] = hi.x & 0xFFFF0000u;
  b[2] = hi.y << 16;
  b[3] = hi.y & 0xFFFF0000u;
}
// Low bytes of 4 values whose bf16 words pack4_bf16 packed into `hi`, packed
// little-endian into one word.
__device__ __forceinline__ uint32_t pack4_lo(const float* v, u32x2 hi) {
  uint32_t b[4];
  hi_bits4(hi, b);
  return lo_byte(v[0], b[0]) | (lo_byte(v[1], b[1]) << 8) | (lo_byte(v[2], b[2]) << 16) |
         (lo_byte(v[3], b[3]) << 24);
}
// The 4 values of a (hi, lo) pair: bf16 words packed as by pack4_bf16, low
// bytes packed as by pack4_lo.
__device__ __forceinline__ void unpack4_hilo(u32x2 hi, uint32_t lo, float* v) {
  uint32_t b[4];
  hi_bits4(hi, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = with_lo(b[e], lo, e);
}


// Tiled layout of the bf16 path's X (both copies), X's low bytes, A and B:
// the matrix (rows multiple of 128, ncols multiple of 32) is stored as tiles
// of 128 rows x 32 columns, each tile contiguous (row-major inside), tiles
// ordered row block by row block.  A 32-column K slab of a 128-row panel is
// then one contiguous 8 KiB (bf16) tile, and any 32 x 32 block 2 KiB.  The
// element offset of (i, j):
__device__ __forceinline__ uint32_t tiled(uint32_t i, uint32_t j, uint32_t ncols) {
  return ((i >> 7) * (ncols >> 5) + (j >> 5)) * 4096u + (i & 127u) * 32u + (j & 31u);
}

// Operand copy of X_t (ping-pong by parity).  A select, not an index, keeps
// the by-value descriptor in registers.
__device__ __forceinline__ void* xbuf(const DevMat& d, int t) { return (t & 1) ? d.xo[1] : d.xo[0]; }

// Operand slabs go from HBM straight into LDS (gfx950 buffer_load_dwordx4
// ... lds): each wave instruction moves 64 x 16 bytes into 1 KiB of
// contiguous LDS, lane l to byte 16 l, so the LDS swizzle is applied by
// choosing which global 16-byte chunk each lane fetches.  A buffer resource
// per slab lives in scalar registers; an empty resource (valid == false)
// issues the instructions without touching memory, which keeps the wait
// counts of the pipeline static.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
#define MUON_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define MUON_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// Workgroup barrier that is also a compiler memory barrier, without the
// fence that would make the compiler wait for every LDS-bound load.
#define MUON_BARRIER() asm volatile("s_barrier" ::: "memory")


__device__ __forceinline__ int xswz(int k) { return 4 * (k & 3); }

// Two bf16 X-layout fragments (columns base + 0..31 and base + 32..63) for
// K step ks.  The four transposing reads and their wait sit in one asm
// block: the compiler would otherwise wait for every in-flight
// direct-to-LDS load before each of them.
__device__ __forceinline__ void frags_x16(u32x4 (&f)[2], const char* l, int base, int lane, int ks) {
  const int g = lane >> 4, r = lane & 15;
  uint32_t addr[2][2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int jel = base + n * 32 + 16 * (g & 1) + 4 * (r & 3);  // first of 4 columns
    const int cb = (jel * 2) >> 4, half = ((jel * 2) >> 3) & 1;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int k = 16 * ks + 8 * (g >> 1) + 4 * m + (r >> 2);
      addr[n][m] = (uint32_t)(uintptr_t)(l + k * 256 + ((cb ^ xswz(k)) << 4) + (half << 3));
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


__device__ __forceinline__ u32x4 pack8_bf16(const float* v) {
  const u32x2 a = pack4_bf16(v[0], v[1], v[2], v[3]), b = pack4_bf16(v[4], v[5], v[6], v[7]);
  return u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void unpack8_bf16(u32x4 r, float* v) {
  unpack4_bf16(u32x2{r.x, r.y}, v);
  unpack4_bf16(u32x2{r.z, r.w}, v + 4);
}
__device__ __forceinline__ u32x2 lo8(const float* v, u32x4 hi) {
  return u32x2{pack4_lo(v, u32x2{hi.x, hi.y}), pack4_lo(v + 4, u32x2{hi.z, hi.w})};
}


// LDS-only workgroup barrier: waits for this wave's LDS operations, not for
// its in-flight direct-to-LDS loads or global stores.
#define MUON_LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

constexpr int kHiLo = 1, kLast = 2, kWriteLo = 4;

// First table entry at or after q (stepping by `stride`) that is not a null
// tile; the entry comes back as its 64-bit word (mat | ti << 16 | tj << 32).
__device__ __forceinline__ int next_entry(const StageArgs& args, int q, int stride, uint64_t& raw) {
  for (; q < args.ntiles; q += stride) {
    raw = *(const MUON_CONST uint64_t*)(const void*)(args.tiles + q);
    if ((raw & 0xFFFFu) != kNullMat) break;
  }
  return q;
}
__device__ __forceinline__ Tile tile_of(uint64_t raw) {
  Tile t;
  t.mat = (uint16_t)raw;
  t.ti = (uint16_t)(raw >> 16);
  t.tj = (uint16_t)(raw >> 32);
  t.pad = 0;
  return t;
}


}  // namespace muon
