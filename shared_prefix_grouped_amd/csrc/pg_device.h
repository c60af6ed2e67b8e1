// Device helpers for the gfx950 (CDNA4) kernels of libpg_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pg {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Initial running max of a row (base-2 domain).  Finite, so that m - m_new and
// fma(s, c, -m) never meet inf - inf; masked scores are -inf and give
// probability exactly 0.
constexpr float kMasked = -1.0e30f;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).
// Operand lanes: A row m = lane % 32, B column n = lane % 32; the 8 k values a
// lane supplies are indexed by (lane / 32, slot) identically for A and B, so
// any assignment of the contraction index to (lane / 32, slot) that both
// operands share gives the same product.
// Result: register r of lane l holds D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 result held by register r in lane half `hi` (= lane / 32).
__device__ __forceinline__ constexpr int mfma_row(int r, int hi) {
  return 8 * (r >> 2) + 4 * hi + (r & 3);
}

// A transposed tile stored in LDS keeps, inside every 16-wide block of the
// contraction index, position u at u with bits 2 and 3 swapped.  Then the 8
// contraction values that lane half `hi` needs for one MFMA k-step (which are
// mfma_row(sub * 8 + j, hi) for j = 0..7, i.e. offsets {0..3, 8..11} + 4 * hi)
// sit contiguously at positions 8 * hi + j, and one 16-byte LDS read fetches
// them.
__device__ __forceinline__ constexpr int swap23(int u) {
  return (u & ~12) | ((u & 4) << 1) | ((u & 8) >> 1);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// One MFMA operand fragment read transposed from a row-major LDS tile
// T[k][m] (m contiguous, row stride `stride` elements), with gfx950's
// ds_read_b64_tr_b16.  The lane receives column m0 + lane % 32 and, in its 8
// slots, rows kb + {0..3, 8..11} + 4 * (lane / 32) -- the same contraction
// order in which a 32x32 accumulator holds its rows (mfma_row), so the
// fragment pairs with P^T / dS^T / P / dS taken straight from accumulator
// registers.
// The instruction works on 16-lane groups: source lane s of a group supplies
// the 8-byte chunk at row k + s / 4, columns c + 4 * (s % 4); lane i of the
// group receives column c + i of rows k .. k + 3 (checked on the GPU).
__device__ __forceinline__ bf16x8 lds_tr_frag(const bf16 *T, int stride, int kb, int m0, int lane) {
  const int s = lane & 15;
  const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int row = kb + 4 * (lane >> 5) + (s >> 2);
  const bf16 *p = T + row * stride + col;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 8 * stride));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Swizzled row-major bf16 tiles in LDS.  A tile of rows with D columns is
// stored without padding; inside each row the 16-byte chunk c lives at chunk
// position c ^ swz_chunk(row).  The permutation makes both access patterns of
// the kernels bank-conflict free (64 banks of 4 bytes):
//   * MFMA operand rows: 16 consecutive rows read at the same column, 16 bytes
//     per lane -> 16 distinct chunk positions (swz_chunk is a bijection on 16
//     consecutive rows);
//   * transposing reads: 4 consecutive rows (first row a multiple of 4) x 64
//     contiguous bytes per half-wave -> the 4 rows land in disjoint 64-byte
//     bank groups (D = 128: swz_chunk varies in bits 2-3 with row % 4; D = 64:
//     rows of equal parity differ in bit 2).
template <int D>
__device__ __forceinline__ int swz_chunk(int r) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  if constexpr (D == 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of (row r, column c) in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return r * D + ((((c >> 3) ^ swz_chunk<D>(r))) << 3) + (c & 7);
}

// 16-byte MFMA operand row fragment (8 consecutive columns starting at c).
template <int D>
__device__ __forceinline__ bf16x8 lds_row_frag(const bf16 *T, int r, int c) {
  return *reinterpret_cast<const bf16x8 *>(T + swz<D>(r, c));
}

// lds_tr_frag for a swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_frag_swz(const bf16 *T, int kb, int m0, int lane) {
  const int s = lane & 15;
  const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const int row = kb + 4 * (lane >> 5) + (s >> 2);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(T + swz<D>(row, col)));
  const bf16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(T + swz<D>(row + 8, col)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __attribute__((address_space(3))) char lds_char;

// gfx950 direct global->LDS copies (global_load_lds_dword / _dwordx4): lane i
// of the wave writes its 4 / 16 bytes at byte 4 i / 16 i of the LDS block
// whose address is in M0 (checked on the GPU).  They are issued through
// inline asm so that the compiler does not treat them as aliasing every later
// LDS read (it would then wait for them before the first read of the *other*
// buffer and serialise the double buffering).  Completion is tracked by
// vmcnt: wait_async_loads() before the barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(const void *g, const void *lds_block) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char *)lds_block);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(a), "v"(g) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void *g, const void *lds_block) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char *)lds_block);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(a), "v"(g) : "memory");
}

// Asynchronous copy of rows [r0, r0 + ROWS) of one head of a row-major bf16
// matrix (D columns at `src`, `row_stride` elements between rows) into a
// swizzled LDS tile.  One wave instruction moves 1 KB; lane i fetches the
// global chunk that the swizzle puts at byte 16 i of the block.  Rows past
// `r_last` are clamped to it (finite data that the caller masks).
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void async_tile_load(bf16 *tile, const bf16 *src, size_t row_stride,
                                                int r0, int r_last, int wave, int lane) {
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per wave instruction
  constexpr int NI = ROWS / RPI; // wave instructions per tile
  static_assert(ROWS % RPI == 0 && NI % NWAVES == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int k = 0; k < NI / NWAVES; ++k) {
    const int i = k * NWAVES + wave;
    const int row = i * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz_chunk<D>(row);
    const int gr = min(r0 + row, r_last);
    lds_dma16(src + (size_t)gr * row_stride + c * 8, tile + i * 512);
  }
}

// The same copy as async_tile_load with addressing hoisted out of the chunk
// loop: each lane's byte offset inside a tile (row * row stride + swizzled
// chunk) is computed once, and an in-bounds tile is copied with the
// scalar-base form of the instruction (64-bit base in SGPRs + 32-bit lane
// offset), so the per-chunk cost is scalar arithmetic only.  Tiles that reach
// past the last row take the clamped per-lane path of async_tile_load.
template <int D, int ROWS, int NWAVES>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NI = ROWS / RPI;
  static constexpr int PER_WAVE = NI / NWAVES;
  static_assert(ROWS % RPI == 0 && NI % NWAVES == 0, "tile must split evenly over the waves");
  uint32_t voff[PER_WAVE];

  __device__ __forceinline__ void init(size_t row_stride, int wave, int lane) {
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int i = k * NWAVES + wave;
      const int row = i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz_chunk<D>(row);
      voff[k] = (uint32_t)(row * row_stride * sizeof(bf16) + c * 16);
    }
  }

  // rows [r0, r0 + ROWS) of src (one head, `row_stride` elements per row)
  // into `tile`, whose LDS byte address is `tile_lds` (see lds_address)
  __device__ __forceinline__ void issue(bf16 *tile, uint32_t tile_lds, const bf16 *src,
                                        size_t row_stride, int r0, int r_last, int wave,
                                        int lane) const {
    if (r0 + ROWS - 1 <= r_last) {
      const uint64_t base = (uint64_t)(uintptr_t)(src + (size_t)r0 * row_stride);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
      const uint64_t sbase = ((uint64_t)hi << 32) | lo;
#pragma unroll
      for (int k = 0; k < PER_WAVE; ++k) {
        const uint32_t a = tile_lds + (uint32_t)((k * NWAVES + wave) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(a), "v"(voff[k]),
                     "s"(sbase)
                     : "memory");
      }
    } else {
      async_tile_load<D, ROWS, NWAVES>(tile, src, row_stride, r0, r_last, wave, lane);
    }
  }
};

// Asynchronous copy of 64 consecutive floats src[min(i, n_last)] (i = 0..63)
// into dst[0..63] by one wave.
__device__ __forceinline__ void async_row_load64(float *dst, const float *src, int n_last, int lane) {
  lds_dma4(src + min(lane, n_last), dst);
}

// s_waitcnt vmcnt(0), leaving the other counters alone: this wave's global
// loads, including the direct-to-LDS ones, have completed.
__device__ __forceinline__ void wait_async_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 3]: all but this wave's n
// most recently issued global loads have completed (loads complete in order).
__device__ __forceinline__ void wait_async_loads_leaving(int n) {
  if (n >= 3) {
    __builtin_amdgcn_s_waitcnt(0x0F73);
  } else if (n == 2) {
    __builtin_amdgcn_s_waitcnt(0x0F72);
  } else if (n == 1) {
    __builtin_amdgcn_s_waitcnt(0x0F71);
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// Work item of a block in a grid of n_tiles x Hq blocks, one per (tile, query
// head).  Workgroups are dispatched to the 8 XCDs round-robin by block index
// and each XCD has its own L2; when the kv heads split evenly over the XCDs,
// all query heads of one kv head are placed on the same XCD, so the K/V rows
// they share stay in one L2.  Within an XCD, blocks go tile by tile in the
// planner's (longest-first) order.
__device__ __forceinline__ void xcd_qhead_work(int bid, int Hq, int Hkv, int &tile, int &h) {
  if ((Hkv & 7) == 0) {
    const int rep = Hq / Hkv;
    const int per = Hq >> 3;  // query heads served by one XCD
    const int xcd = bid & 7, slot = bid >> 3;
    tile = slot / per;
    const int j = slot - tile * per;
    const int gi = j / rep;
    h = (xcd + 8 * gi) * rep + (j - gi * rep);
  } else {
    tile = bid / Hq;
    h = bid - tile * Hq;
  }
}

// Same for a grid of n_tiles x Hkv blocks, one per (tile, kv head).
__device__ __forceinline__ void xcd_kvhead_work(int bid, int Hkv, int &tile, int &hk) {
  if ((Hkv & 7) == 0) {
    const int per = Hkv >> 3;
    const int xcd = bid & 7, slot = bid >> 3;
    tile = slot / per;
    hk = xcd + 8 * (slot - tile * per);
  } else {
    tile = bid / Hkv;
    hk = bid - tile * Hkv;
  }
}

// Raw buffer resource (stride 0) over `bytes` (< 2^32) bytes at `p`, for
// buffer loads with a scalar descriptor.  The range check covers the vector
// offset plus the instruction offset only: a load whose vector + immediate
// offset is at or past `bytes` returns zero and reads nothing, while the
// scalar offset is added unchecked, so it must keep every in-range access
// inside the tensor by itself.  Word 3 is the gfx9-family raw-buffer format
// (32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_resource(const void *p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0,
                                           (int)(uint32_t)bytes, 0x00020000);
}

// An empty asm that claims to read and rewrite x: a load into x is complete
// before it (the wait is inserted there), so the load cannot sink below a
// preceding s_waitcnt, and no use of x moves above it.
template <typename Tv>
__device__ __forceinline__ void pin(Tv &x) {
  asm volatile("" : "+v"(x));
}
template <typename Tv, int N>
__device__ __forceinline__ void pin(Tv (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) pin(x[i]);
}

typedef __attribute__((address_space(1))) const char gbl_cchar;
typedef __attribute__((address_space(1))) const bf16x8 gbl_bf16x8;

// A wave-uniform global pointer, as a global-address-space byte pointer held
// in scalar registers (so that `uniform_ptr(p) + lane_offset` compiles to the
// scalar-base form of a global load).
__device__ __forceinline__ gbl_cchar *uniform_ptr(const void *p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (gbl_cchar *)(((uint64_t)hi << 32) | lo);
}

// Byte address of an LDS array in the LDS aperture (for M0), as a scalar.
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_char *)p);
}

// Index of the calling wave in its workgroup, as a scalar (so that per-wave
// decisions compile to scalar branches).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// MFMA operand fragments from a swizzled tile with the lane-dependent part of
// the address computed once.  swz_chunk depends only on row % 16, so moving a
// fragment by a multiple of 16 rows only adds row * D * 2 bytes, which the
// compiler folds into the LDS instruction's immediate offset.
template <int D>
struct SwzFrags {
  uint32_t row_off[D / 16];     // row l32, columns 16 st + 8 hi .. + 8
  uint32_t tr_off[D / 32][2];   // transposing reads: see lds_tr_frag_swz

  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hi = lane >> 5, s = lane & 15;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) row_off[st] = 2 * swz<D>(l32, st * 16 + hi * 8);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      const int col = nb * 32 + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
      const int row = 4 * hi + (s >> 2);
      tr_off[nb][0] = 2 * swz<D>(row, col);
      tr_off[nb][1] = 2 * swz<D>(row + 8, col);
    }
  }
  // Move every offset to the other half of a double buffer of `bytes` per
  // half (a power of two above every offset's tile part): the buffer choice
  // then lives in the offsets, and the tile base stays a constant.
  __device__ __forceinline__ void flip(uint32_t bytes) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) row_off[st] ^= bytes;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      tr_off[nb][0] ^= bytes;
      tr_off[nb][1] ^= bytes;
    }
  }
  // rows r0 + l32 (r0 a multiple of 16), 8 columns at 16 st + 8 hi
  __device__ __forceinline__ bf16x8 row(lds_cchar *tile, int r0, int st) const {
    return *reinterpret_cast<lds_bf16x8 *>(tile + row_off[st] + r0 * D * 2);
  }
  // lds_tr_frag_swz(tile, kb, 32 nb, lane), kb a multiple of 16
  __device__ __forceinline__ bf16x8 tr(lds_cchar *tile, int kb, int nb) const {
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(tile + tr_off[nb][0] + kb * D * 2));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4 *)(tile + tr_off[nb][1] + kb * D * 2));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// An LDS array as an address-space-3 byte pointer.
__device__ __forceinline__ lds_cchar *lds_bytes(const void *p) { return (lds_cchar *)p; }

// The values of x in lanes l mod 32 and l mod 32 + 32, in every lane l, in
// that order: v_permlane32_swap exchanges the upper half of one register with
// the lower half of another without going through the LDS.  Both halves then
// combine the same two values in the same order.
__device__ __forceinline__ void wave_halves(float x, float &lo, float &hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Pack 8 floats (registers r0..r0+7 of a 32x32 result) into bf16x8.
__device__ __forceinline__ bf16x8 pack8(const f32x16 &s, int r0) {
  bf16x8 p;
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = (__bf16)s[r0 + j];
  return p;
}

__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(uint32_t(u) << 16);
}

}  // namespace pg
