// The products of the response log-probability head (skillsmp.com
// "prefix-grouper-grpo", "Step 4: Training Integration with GRPO": per scored
// row, log-softmax of the logits over the vocabulary, gathered at the next
// token), all on one MFMA tile kernel: C = A B^T for bf16 matrices A [M, K]
// and B [N, K] stored row-major (both contiguous along the contraction), fp32
// accumulation, one 256 x 256 tile of C per workgroup.
//
// The logits Z = H_pred W^T are computed as their transpose (A = W, B =
// H_pred), so that lane l32 of an MFMA result is a scored row and its 16
// registers are vocab entries; the log-softmax then works in place and the
// [n, V] logits never reach HBM:
//   forward (EPI_LSE):    per scored row, the tile's max and sum of
//                         exp(z - max); a second kernel combines the per-tile
//                         pairs of a row into lse = max + log(sum), computes
//                         the target logit z[token] as one dot product, and
//                         logp = z[token] - lse;
//   backward (EPI_GRAD):  G[k, v] = dlogp[k] ([v == token_k] - exp(z - lse_k)),
//                         the gradient of the loss with respect to the logits
//                         (the token entries by a second kernel), stored as
//                         bf16 twice: G [n, V64] and G^T [V, n64]
//                         (V64, n64: rounded up to multiples of 64, pad zero,
//                         so that rows start on 128-byte lines);
//   products (EPI_STORE): dH_pred = G W as G [n, V64] . (W^T [dm, V64])^T and
//                         dW = G^T H_pred as G^T [V, n64] . (H_pred^T [dm, n64])^T
//                         over the first round8(V) / round8(n) contraction
//                         entries, stored as fp32.
// Every reduction has a fixed order: results are bitwise repeatable.

#include <type_traits>

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

constexpr int HT = 256;    // tile of C: A rows and B rows
constexpr int HK = 64;     // contraction block
constexpr int HWAVES = 4;  // 2 x 2 waves of 128 x 128
constexpr float kLog2e = 1.4426950408889634f;

enum { EPI_LSE = 0, EPI_GRAD = 1, EPI_STORE = 2 };

// XOR swizzle of the 16-byte chunks of a 64-element (128-byte) LDS row, as in
// the attention tiles: conflict-free 16-byte reads of 16 consecutive rows at
// one column, and it depends on row % 16 only.
__device__ __forceinline__ int hswz(int r) { return swz_chunk<64>(r); }

// Tile (A tile ta, B tile tb) of workgroup `bid`.  Workgroups go to the 8
// XCDs round-robin by index; the map hands each XCD one contiguous run of a
// raster that walks bands of 8 B tiles, A tile by A tile, so the ~32 tiles an
// XCD holds at once share 4 A tiles and 8 B tiles in its L2.
__device__ __forceinline__ void tile_of(int bid, int total, int nta, int ntb, int &ta, int &tb) {
  const int q = total >> 3, rem = total & 7;
  const int x = bid & 7, s = bid >> 3;
  const int o = (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + s;
  const int band = o / (nta * 8);
  const int b0 = band * 8;
  const int wb = min(8, ntb - b0);
  const int j = o - band * nta * 8;
  ta = j / wb;
  tb = b0 + j - (j / wb) * wb;
}

struct NtArgs {
  const bf16 *a, *b;  // [M, K] and [N, K], row strides lda, ldb (multiples of 8)
  int M, N, K, lda, ldb;
  // EPI_LSE / EPI_GRAD (A = W [V, dm], B = H_pred [n, dm]: M = V, N = n)
  const int32_t *scored_row;  // [n] target row of each scored entry
  const int32_t *tokens;      // [T] token ids of the packed rows
  float *part_m, *part_s;     // EPI_LSE: [M tiles, n] per-tile max and sum
  const float *lse, *dlogp;   // EPI_GRAD: [n]
  bf16 *g, *gt;               // EPI_GRAD: [n, ldg] and [V, ldgt]
  int ldg, ldgt;              // V64, n64
  float *c;                   // EPI_STORE: [M, ldc]
  int ldc;
};

// Direct global->LDS copies of the two 256 x 64 tiles of one contraction
// block.  Instruction i (= 4 k + wave) of a tile moves rows 8 i .. 8 i + 7;
// lane L writes LDS bytes 16 L of that 1 KB block, i.e. row 8 i + L / 8 at
// chunk position L % 8, and so fetches the chunk that the swizzle puts there.
// Rows past the last one are clamped to it (finite values that the epilogues
// never store).  In a contraction block that reaches past K, chunks past it
// are fetched from chunk 0 of the block instead (in bounds; the fragments
// they feed are zeroed before use).
struct NtCopy {
  uint32_t off[16];  // byte offset of the lane's chunk in block 0: A rows (k < 8), B rows
  int chunk;         // lane's source chunk in the block

  // (row % 16 = 8 (wave % 2) + lane / 8 for every k, so the chunk is one per lane)
  __device__ __forceinline__ void init(const NtArgs &p, int i0, int j0, int wave, int lane) {
    chunk = (lane & 7) ^ hswz(8 * wave + (lane >> 3));
    // (the host keeps M lda 2 and N ldb 2 under 2^32)
    const uint32_t ra = (uint32_t)p.lda * 2u, rb = (uint32_t)p.ldb * 2u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = (k * HWAVES + wave) * 8 + (lane >> 3);
      off[k] = (uint32_t)min(i0 + row, p.M - 1) * ra + (uint32_t)(chunk * 16);
      off[8 + k] = (uint32_t)min(j0 + row, p.N - 1) * rb + (uint32_t)(chunk * 16);
    }
  }

  // Addresses of contraction block kb into the buffers at LDS byte addresses
  // la / lb.  Scalar 64-bit bases: uniform_ptr zero-extends the low word
  // (readfirstlane returns int; a sign-extended low word would corrupt the
  // high one).  In a block that K cuts, a chunk at or past K reads chunk 0 of
  // the block instead.
  struct Block {
    uint64_t sa, sb;
    uint32_t fix, la, lb;
  };
  __device__ __forceinline__ Block block(const NtArgs &p, int kb, uint32_t la, uint32_t lb) const {
    Block b;
    b.sa = (uint64_t)(uintptr_t)uniform_ptr(p.a + (size_t)kb * HK);
    b.sb = (uint64_t)(uintptr_t)uniform_ptr(p.b + (size_t)kb * HK);
    b.fix = kb * HK + chunk * 8 >= p.K ? (uint32_t)(chunk * 16) : 0u;
    b.la = la;
    b.lb = lb;
    return b;
  }

  // copy instruction k (0..15) of a block: 1 KB of A (k < 8) or of B
  template <int k>
  __device__ __forceinline__ void one(const Block &b, int wave) const {
    const uint32_t a = (k < 8 ? b.la : b.lb) + (uint32_t)(((k & 7) * HWAVES + wave) * 1024);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(a),
                 "v"(off[k] - b.fix), "s"(k < 8 ? b.sa : b.sb)
                 : "memory");
  }
  template <int k = 0>
  __device__ __forceinline__ void all(const Block &b, int wave) const {
    one<k>(b, wave);
    if constexpr (k + 1 < 16) all<k + 1>(b, wave);
  }
};

__device__ __forceinline__ bf16x8 lds_frag(lds_cchar *tile, uint32_t off) {
  return *reinterpret_cast<lds_bf16x8 *>(tile + off);
}

template <int EPI>
__global__ __launch_bounds__(HWAVES * 64) void nt_tile_kernel(NtArgs p, int nta, int ntb) {
  // operand buffers: A (2 x 32 KB) then B (2 x 32 KB); after the main loop
  // EPI_GRAD stages the tile's 256 x 256 bf16 gradient in the same 128 KB
  __shared__ __attribute__((aligned(16))) bf16 sAB[4 * HT * HK];
  bf16 *const sA = sAB, *const sB = sAB + 2 * HT * HK;
  __shared__ float red_m[EPI == EPI_LSE ? 2 : 1][HT], red_s[EPI == EPI_LSE ? 2 : 1][HT];

  int ta, tb;
  tile_of(blockIdx.x, nta * ntb, nta, ntb, ta, tb);
  const int i0 = ta * HT, j0 = tb * HT;  // first A row and B row of the tile
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int l32 = lane & 31, hi = lane >> 5;
  const int wa = wave & 1, wb = wave >> 1;  // A half, B half of the tile
  const int K = p.K;
  const int nkb = (K + HK - 1) / HK;  // 64-deep contraction blocks, the last maybe partial
  const bool tail = (K % HK) != 0;

  NtCopy cp;
  cp.init(p, i0, j0, wave, lane);
  const uint32_t la = lds_address(sA), lb = lds_address(sB);
  constexpr uint32_t BUF = HT * HK * 2;  // bytes per buffer of one tile

  // fragment offsets: row l32 (+ 32 a + 128 half), chunk 2 st + hi
  uint32_t foff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) foff[st] = (uint32_t)(l32 * 128 + (((2 * st + hi) ^ hswz(l32)) << 4));

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  lds_cchar *const ta0 = lds_bytes(sA) + wa * 128 * 128;
  lds_cchar *const tb0 = lds_bytes(sB) + wb * 128 * 128;
  struct Frags {
    bf16x8 a[4], b[4];
  };
  // fragment i (0..7: A 0..3, B 0..3) of 16-deep step st of the block in buffer `cur`
  auto frag = [&](uint32_t cur, int st, int i) {
    return lds_frag((i < 4 ? ta0 : tb0) + cur + (i & 3) * 32 * 128, foff[st]);
  };
  auto load = [&](Frags &f, uint32_t cur, int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = frag(cur, st, i);
      f.b[i] = frag(cur, st, 4 + i);
    }
  };
  auto mma = [&](const Frags &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(f.a[i], f.b[j], acc[i][j]);
  };
  // the 16 MFMAs of one step with the 8 fragment reads of the next one
  // spread between them (one read per two MFMAs)
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    }
  };
  // Step 3 of a block after the barrier, with the 16 copy instructions of
  // block kb + 2 (if any) and the 8 fragment reads of the next block's step 0
  // (if it is a whole block) placed one per MFMA: issued in one burst they
  // would leave the MFMA pipe idle.  The MFMAs are unconditional (the
  // accumulators take one path through the loop); only the copies and reads
  // are.
  auto step3 = [&](const Frags &f, Frags &g, const NtCopy::Block &blk, bool cp_ok, bool rd_ok,
                   uint32_t nxt) {
#define PG_NT_SLOT(k)                                                                      \
  acc[(k) >> 2][(k) & 3] = mfma32(f.a[(k) >> 2], f.b[(k) & 3], acc[(k) >> 2][(k) & 3]);    \
  if (cp_ok) cp.one<k>(blk, wave);                                                         \
  if (((k) & 1) && rd_ok) {                                                                \
    constexpr int i = (k) >> 1;                                                            \
    if (i < 4)                                                                             \
      g.a[i & 3] = frag(nxt, 0, i);                                                        \
    else                                                                                   \
      g.b[i & 3] = frag(nxt, 0, i);                                                        \
  }
    PG_NT_SLOT(0) PG_NT_SLOT(1) PG_NT_SLOT(2) PG_NT_SLOT(3)
    PG_NT_SLOT(4) PG_NT_SLOT(5) PG_NT_SLOT(6) PG_NT_SLOT(7)
    PG_NT_SLOT(8) PG_NT_SLOT(9) PG_NT_SLOT(10) PG_NT_SLOT(11)
    PG_NT_SLOT(12) PG_NT_SLOT(13) PG_NT_SLOT(14) PG_NT_SLOT(15)
#undef PG_NT_SLOT
  };

  // Whole 64-deep blocks, two in flight: block kb + 2 is copied into the
  // buffer of block kb once every wave holds block kb's last fragments in
  // registers (the barrier between its steps 2 and 3), and block kb + 1's
  // first fragments are read while step 3 of block kb multiplies.
  const int nfull = K / HK;
  if (nkb > 0) cp.all(cp.block(p, 0, la, lb), wave);
  if (nkb > 1) {
    cp.all(cp.block(p, 1, la + BUF, lb + BUF), wave);
    // each wave issues 16 copies per block: vmcnt(16) waits for block 0's
    // and leaves block 1's in flight
    __builtin_amdgcn_s_waitcnt(0x0F70 | (1 << 14));
  } else {
    wait_async_loads();
  }
  __syncthreads();
  Frags f0, f1;
  if (nfull > 0) load(f0, 0, 0);
  for (int kb = 0; kb < nfull; ++kb) {
    const uint32_t cur = (kb & 1) * BUF, nxt = BUF - cur;
    load(f1, cur, 1);
    mma(f0);
    interleave();
    load(f0, cur, 2);
    mma(f1);
    interleave();
    load(f1, cur, 3);
    mma(f0);
    interleave();
    wait_async_loads();
    __syncthreads();  // block kb + 1 is in LDS; block kb's reads are done
    step3(f1, f0, cp.block(p, kb + 2, la + cur, lb + cur), kb + 2 < nkb, kb + 1 < nfull, nxt);
  }
  if (tail) {
    // the last, partial block (in LDS since the last barrier): a lane's 8
    // contraction values at or past K are zeroed in both operands.  All
    // fragments are read first and the four steps run with no branch around
    // the MFMAs (a data-dependent step count made the compiler copy the 256
    // accumulators out and back); EPI_GRAD then reuses the operand buffers,
    // so every wave's reads end at a barrier before its MFMAs.
    const uint32_t cur = (nfull & 1) * BUF;
    const int rest = K - nfull * HK;  // 8 .. 56
    Frags ft[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      load(ft[st], cur, st);
      const bool ok = 16 * st + 8 * hi < rest;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ft[st].a[i] = ok ? ft[st].a[i] : bf16x8{};
        ft[st].b[i] = ok ? ft[st].b[i] : bf16x8{};
      }
    }
    if constexpr (EPI == EPI_GRAD) __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; ++st) mma(ft[st]);
  }

  // register r of block a / lane column b: A row ib + 32 a + mfma_row(r, hi),
  // B row jb + 32 b + l32
  const int ib = i0 + wa * 128, jb = j0 + wb * 128;
  if constexpr (EPI == EPI_LSE) {
    // per scored row of the wave: max and sum of exp(z - max) over its 128
    // vocab entries (64 in the lane, 64 in its partner in the other half of
    // the wave); with kMask, entries past the vocabulary (the last vocab
    // tile) take no part, and a slab wholly past it gives max -inf, sum 0
    auto rows = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
      auto val = [&](int a, int b, int r) {
        const float z = acc[a][b][r];
        if constexpr (kMask) return ib + 32 * a + mfma_row(r, hi) < p.M ? z : -INFINITY;
        return z;
      };
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float m4[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float x = val(a, b, 0);
#pragma unroll
          for (int r = 1; r < 16; ++r) x = fmaxf(x, val(a, b, r));
          m4[a] = x;
        }
        float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        float lo, up;
        wave_halves(mx, lo, up);
        mx = fmaxf(lo, up);
        const float ml = mx == -INFINITY ? 0.f : mx * kLog2e;
        float s4[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float x = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) x += fast_exp2(fmaf(val(a, b, r), kLog2e, -ml));
          s4[a] = x;
        }
        float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        wave_halves(sum, lo, up);
        sum = lo + up;
        const int rl = wb * 128 + b * 32 + l32;  // row inside the tile
        if (hi == 0) {
          red_m[wa][rl] = mx;
          red_s[wa][rl] = sum;
        }
      }
    };
    if (i0 + HT <= p.M)
      rows(std::false_type{});
    else
      rows(std::true_type{});
    __syncthreads();
    // the two vocab halves of each row, in order
    for (int rl = threadIdx.x; rl < HT; rl += HWAVES * 64) {
      const int row = j0 + rl;
      if (row >= p.N) continue;
      const float ma = red_m[0][rl], mb = red_m[1][rl];
      const float m = fmaxf(ma, mb);
      const float sum = red_s[0][rl] * fast_exp2((ma - m) * kLog2e) +
                        red_s[1][rl] * fast_exp2((mb - m) * kLog2e);
      p.part_m[(size_t)ta * p.N + row] = m;
      p.part_s[(size_t)ta * p.N + row] = sum;
    }
  } else if constexpr (EPI == EPI_GRAD) {
    // scored row k = jb + 32 b + l32 and vocab entries v = ib + 32 a +
    // mfma_row(r, hi): G[k, v] = -dlogp[k] exp(z - lse[k]) here, with no
    // branch (one path keeps the accumulators in place); the token's entry,
    // dlogp[k] (1 - exp(z_token - lse[k])), is written afterwards by
    // head_grad_token_kernel.  The values go to LDS first ([256 rows][256
    // entries] bf16, 16-byte chunk c of tile row r at chunk position
    // c ^ gswz(r)), so that both G [n, V64] and G^T [V, n64] leave in whole
    // 16-byte chunks of consecutive entries.  The pad rows n <= k < n64 of
    // G^T and the pad entries V <= v < V64 of G are written as zeros: tiles
    // start at multiples of 256, so the tiles that hold row n - 1 and entry
    // V - 1 also cover the pads.
    const int V = p.M, n = p.N;
    // (r ^ r >> 3) & 31: at most two lanes per bank group both for the
    // staging writes (32 consecutive rows, one chunk) and for the column
    // reads below (rows 8 c + k, c = 0..31, one entry)
    auto gswz = [](int r) { return (r ^ (r >> 3)) & 31; };
    auto gpos = [&](int r, int v) { return r * 512 + (((v >> 3) ^ gswz(r)) << 4) + ((v & 7) << 1); };
    // (no wave reads the operand buffers after the loop's last barrier, or
    // after the tail's: the staging writes may start)
    char *const stg = reinterpret_cast<char *>(sAB);
    auto stage = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;  // the last vocab tile
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int rt = wb * 128 + 32 * b + l32;  // tile row
        const int row = j0 + rt, rc = min(row, n - 1);
        // rows past n: d = 0 with the last row's lse, so every value is 0
        const float ll = p.lse[rc] * kLog2e, nd = row < n ? -p.dlogp[rc] : 0.f;
        int gs = gswz(rt);
        pin(gs);  // (the staging addresses are formed here, not hoisted)
        char *const srow = stg + rt * 512 + hi * 8;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // registers 4 q .. 4 q + 3: vocab entries vq .. vq + 3 (chunk cq)
            const int cq = wa * 16 + 4 * a + q;
            float gv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              gv[j] = nd * fast_exp2(fmaf(acc[a][b][4 * q + j], kLog2e, -ll));
              if constexpr (kMask) gv[j] = i0 + 8 * cq + 4 * hi + j < V ? gv[j] : 0.f;
            }
            *reinterpret_cast<u32x2 *>(srow + ((cq ^ gs) << 4)) =
                pack4_bf16(gv[0], gv[1], gv[2], gv[3]);
          }
      }
    };
    if (i0 + HT <= V)
      stage(std::false_type{});
    else
      stage(std::true_type{});
    __syncthreads();
    const int tid = threadIdx.x;
    // G: 32 consecutive threads write one row's 256 entries (512 bytes)
#pragma unroll 4
    for (int it = 0; it < HT * HT / 8 / (HWAVES * 64); ++it) {
      const int idx = it * HWAVES * 64 + tid, rt = idx >> 5, c = idx & 31;
      const int row = j0 + rt, v0 = i0 + 8 * c;
      if (row < n && v0 < p.ldg)
        *reinterpret_cast<bf16x8 *>(p.g + (size_t)row * p.ldg + v0) =
            *reinterpret_cast<const bf16x8 *>(stg + rt * 512 + ((c ^ gswz(rt)) << 4));
    }
    // G^T: 32 consecutive threads write one vocab entry's 256 rows
#pragma unroll 4
    for (int it = 0; it < HT * HT / 8 / (HWAVES * 64); ++it) {
      const int idx = it * HWAVES * 64 + tid, vt = idx >> 5, c = idx & 31;
      const int v = i0 + vt, r0 = 8 * c, row0 = j0 + r0;
      if (v < V && row0 < p.ldgt) {
        bf16x8 x;
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = *reinterpret_cast<const bf16 *>(stg + gpos(r0 + k, vt));
        *reinterpret_cast<bf16x8 *>(p.gt + (size_t)v * p.ldgt + row0) = x;
      }
    }
  } else {
    // C [M, ldc] fp32: for one register, the 32 lanes of a half store 32
    // consecutive columns
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = ib + 32 * a + mfma_row(r, hi);
        if (i >= p.M) continue;
        float *crow = p.c + (size_t)i * p.ldc;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int j = jb + 32 * b + l32;
          if (j < p.N) crow[j] = acc[a][b][r];
        }
      }
  }
}

// One wave per scored row k: the target logit z[token] = H_pred[k] . W[token]
// (fp32 dot product over d_model, 8 entries per lane and pass, then a xor
// butterfly, so every lane holds the same sum), and lse from the per-tile
// (max, sum) pairs: lane l combines tiles l, l + 64, ... in order, then a xor
// butterfly of the pairs.  Both reductions have a fixed order.
__global__ __launch_bounds__(256) void head_lse_combine_kernel(
    const float *__restrict__ part_m, const float *__restrict__ part_s, const bf16 *__restrict__ hp,
    const bf16 *__restrict__ w, const int32_t *__restrict__ scored_row,
    const int32_t *__restrict__ tokens, float *__restrict__ logp, float *__restrict__ lse, int n,
    int V, int dm, int nvt) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + wave_id();
  if (k >= n) return;
  const int tok = tokens[scored_row[k]];
  const bool tok_ok = (unsigned)tok < (unsigned)V;
  float zt = 0.f;
  if (tok_ok) {
    const bf16x8 *hr = reinterpret_cast<const bf16x8 *>(hp + (size_t)k * dm);
    const bf16x8 *wr = reinterpret_cast<const bf16x8 *>(w + (size_t)tok * dm);
    for (int c = lane; c < dm / 8; c += 64) {
      const bf16x8 x = hr[c], y = wr[c];
#pragma unroll
      for (int j = 0; j < 8; ++j) zt = fmaf((float)x[j], (float)y[j], zt);
    }
  }
  float m = -INFINITY, s = 0.f;
  for (int t = lane; t < nvt; t += 64) {
    const float m2 = part_m[(size_t)t * n + k], s2 = part_s[(size_t)t * n + k];
    const float mn = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * fast_exp2((m - mn) * kLog2e)) + s2 * fast_exp2((m2 - mn) * kLog2e);
    m = mn;
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    zt += __shfl_xor(zt, x);
    const float m2 = __shfl_xor(m, x), s2 = __shfl_xor(s, x);
    const float mn = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * fast_exp2((m - mn) * kLog2e)) +
        (m2 == -INFINITY ? 0.f : s2 * fast_exp2((m2 - mn) * kLog2e));
    m = mn;
  }
  if (lane == 0) {
    const float l = m + __logf(s);
    lse[k] = l;
    logp[k] = tok_ok ? zt - l : __int_as_float(0x7fc00000);  // NaN: bad id
  }
}

// One wave per scored row k: the token entry of the logit gradient,
// G[k, t] = dlogp[k] (1 - exp(z_t - lse[k])) with z_t = H_pred[k] . W[t] (the
// dot product of head_lse_combine_kernel), written into G and G^T over the
// -dlogp[k] exp(z_t - lse[k]) that the tile kernel left there.  Rows whose
// token is outside the vocabulary keep the tile kernel's values.
__global__ __launch_bounds__(256) void head_grad_token_kernel(
    const bf16 *__restrict__ hp, const bf16 *__restrict__ w, const int32_t *__restrict__ scored_row,
    const int32_t *__restrict__ tokens, const float *__restrict__ lse,
    const float *__restrict__ dlogp, bf16 *__restrict__ g, bf16 *__restrict__ gt, int n, int V,
    int dm, int ldg, int ldgt) {
  const int lane = threadIdx.x & 63;
  const int k = blockIdx.x * 4 + wave_id();
  if (k >= n) return;
  const int tok = tokens[scored_row[k]];
  if ((unsigned)tok >= (unsigned)V) return;
  const bf16x8 *hr = reinterpret_cast<const bf16x8 *>(hp + (size_t)k * dm);
  const bf16x8 *wr = reinterpret_cast<const bf16x8 *>(w + (size_t)tok * dm);
  float zt = 0.f;
  for (int c = lane; c < dm / 8; c += 64) {
    const bf16x8 x = hr[c], y = wr[c];
#pragma unroll
    for (int j = 0; j < 8; ++j) zt = fmaf((float)x[j], (float)y[j], zt);
  }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) zt += __shfl_xor(zt, x);
  if (lane == 0) {
    const float d = dlogp[k];
    const bf16 v = (bf16)(d * (1.f - fast_exp2((zt - lse[k]) * kLog2e)));
    g[(size_t)k * ldg + tok] = v;
    gt[(size_t)tok * ldgt + k] = v;
  }
}

// dst [C, ldd] bf16 with dst[c][r] = src[idx(r)][c] for r < R and 0 for
// R <= r < ldd (ldd even), where idx(r) = rows[r] (or r when rows is NULL)
// and src is [*, C] row-major with C a multiple of 8.  64 x 64 tiles through
// LDS, 16-byte global reads and 4-byte global writes.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const bf16 *__restrict__ src,
                                                            const int32_t *__restrict__ rows,
                                                            int R, int C, bf16 *__restrict__ dst,
                                                            int ldd) {
  __shared__ bf16 t[64][64 + 2];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  // read: 64 source rows x 8 chunks of 8 columns
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = tid + it * 256, rr = e >> 3, ch = e & 7;
    const int r = r0 + rr, c = c0 + 8 * ch;
    bf16x8 v = bf16x8{};
    if (r < R && c < C)
      v = *reinterpret_cast<const bf16x8 *>(src + (size_t)(rows ? rows[r] : r) * C + c);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[rr][8 * ch + j] = v[j];
  }
  __syncthreads();
  // write: 64 destination rows (source columns) x 32 pairs of source rows
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int e = tid + it * 256, cc = e >> 5, pr = e & 31;
    const int c = c0 + cc, r = r0 + 2 * pr;
    if (c < C && r < ldd) {
      bf16x2 v;
      v[0] = t[2 * pr][cc];
      v[1] = t[2 * pr + 1][cc];
      *reinterpret_cast<bf16x2 *>(dst + (size_t)c * ldd + r) = v;
    }
  }
}

NtArgs nt_args(const void *a, const void *b, int M, int N, int K, int lda, int ldb) {
  NtArgs x{};
  x.a = (const bf16 *)a;
  x.b = (const bf16 *)b;
  x.M = M;
  x.N = N;
  x.K = K;
  x.lda = lda;
  x.ldb = ldb;
  return x;
}

int tiles(int x) { return (x + HT - 1) / HT; }

template <int EPI>
hipError_t launch_nt(const NtArgs &a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const int nta = tiles(a.M), ntb = tiles(a.N);
  hipLaunchKernelGGL(nt_tile_kernel<EPI>, dim3(nta * ntb), dim3(HWAVES * 64), 0, s, a, nta, ntb);
  return hipGetLastError();
}

}  // namespace

int head_vocab_tiles(int V) { return tiles(V); }

hipError_t launch_head_logprob(const void *hp, const void *w, const int32_t *scored_row,
                               const int32_t *tokens, float *part_m, float *part_s, float *logp,
                               float *lse, int n, int V, int dm, hipStream_t s) {
  if (n == 0) return hipSuccess;
  NtArgs a = nt_args(w, hp, V, n, dm, dm, dm);
  a.scored_row = scored_row;
  a.tokens = tokens;
  a.part_m = part_m;
  a.part_s = part_s;
  hipError_t e = launch_nt<EPI_LSE>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_lse_combine_kernel, dim3((n + 3) / 4), dim3(256), 0, s, part_m, part_s,
                     (const bf16 *)hp, (const bf16 *)w, scored_row, tokens, logp, lse, n, V, dm,
                     tiles(V));
  return hipGetLastError();
}

hipError_t launch_head_grad(const void *hp, const void *w, const int32_t *scored_row,
                            const int32_t *tokens, const float *lse, const float *dlogp, void *g,
                            void *gt, int n, int V, int dm, hipStream_t s) {
  if (n == 0) return hipSuccess;
  NtArgs a = nt_args(w, hp, V, n, dm, dm, dm);
  a.scored_row = scored_row;
  a.tokens = tokens;
  a.lse = lse;
  a.dlogp = dlogp;
  a.g = (bf16 *)g;
  a.gt = (bf16 *)gt;
  a.ldg = round64(V);
  a.ldgt = round64(n);
  hipError_t e = launch_nt<EPI_GRAD>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_grad_token_kernel, dim3((n + 3) / 4), dim3(256), 0, s, (const bf16 *)hp,
                     (const bf16 *)w, scored_row, tokens, lse, dlogp, (bf16 *)g, (bf16 *)gt, n, V,
                     dm, a.ldg, a.ldgt);
  return hipGetLastError();
}

hipError_t launch_nt_f32(const void *a, const void *b, int M, int N, int K, int lda, int ldb,
                         float *c, int ldc, hipStream_t s) {
  NtArgs x = nt_args(a, b, M, N, K, lda, ldb);
  x.c = c;
  x.ldc = ldc;
  return launch_nt<EPI_STORE>(x, s);
}

hipError_t launch_transpose_pad(const void *src, const int32_t *rows, int R, int C, void *dst,
                                int ldd, hipStream_t s) {
  if (C == 0 || ldd == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3((ldd + 63) / 64, (C + 63) / 64), dim3(256), 0, s,
                     (const bf16 *)src, rows, R, C, (bf16 *)dst, ldd);
  return hipGetLastError();
}

}  // namespace pg
