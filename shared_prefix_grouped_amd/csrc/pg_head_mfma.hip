// The logits products of the response log-probability head, with the
// log-softmax work done in the epilogue of the product tiles, so that the
// [n, V] fp32 logits never reach HBM (skillsmp.com "prefix-grouper-grpo",
// "Step 4: Training Integration with GRPO": per scored row, log-softmax over
// the vocabulary, gathered at the next token).
//
// One workgroup computes a 256 (vocab) x 256 (scored rows) tile of
// Z^T = W H_pred^T with bf16 MFMAs and fp32 accumulation, and then
//   forward:  per scored row, the tile's max and sum of exp(z - max) over its
//             vocab entries; a second kernel combines the per-tile (max, sum)
//             pairs of a row into lse = max + log(sum), computes the target
//             logit z[token] as one dot product, and logp = z[token] - lse;
//   backward: G[k, v] = dlogp[k] * ([v == token_k] - exp(z[k, v] - lse[k])),
//             the gradient of the loss with respect to the logits, stored as
//             bf16 for the two plain products dH = G W and dW = G^T H_pred.
// Every reduction has a fixed order: results are bitwise repeatable.
//
// Layout of the product: lane l32 of an MFMA result is a scored row and the
// 16 registers are vocab entries, so a row's values sit in one lane (and its
// partner in the other half of the wave); the row reductions are register
// loops plus one exchange between the wave halves and one between the two
// waves that share the rows.

#include <type_traits>

#include "pg_device.h"
#include "pg_internal.h"

namespace pg {
namespace {

constexpr int HT = 256;    // tile: vocab entries and scored rows
constexpr int HK = 64;     // contraction block (d_model)
constexpr int HWAVES = 4;  // 2 x 2 waves of 128 x 128
constexpr float kLog2e = 1.4426950408889634f;

// XOR swizzle of the 16-byte chunks of a 64-element (128-byte) LDS row, as in
// the attention tiles: conflict-free 16-byte reads of 16 consecutive rows at
// one column, and it depends on row % 16 only.
__device__ __forceinline__ int hswz(int r) { return swz_chunk<64>(r); }

// Tile (vocab tile vt, row tile mt) of workgroup `bid`.  Workgroups go to the
// 8 XCDs round-robin by index; the map hands each XCD one contiguous run of a
// raster that walks bands of 8 row tiles, vocab tile by vocab tile, so the
// ~32 tiles an XCD holds at once share 4 W tiles and 8 H_pred tiles in its L2.
__device__ __forceinline__ void head_tile_of(int bid, int total, int nvt, int nmt, int &vt,
                                             int &mt) {
  const int q = total >> 3, rem = total & 7;
  const int x = bid & 7, s = bid >> 3;
  const int o = (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + s;
  const int band = o / (nvt * 8);
  const int b0 = band * 8;
  const int wb = min(8, nmt - b0);
  const int j = o - band * nvt * 8;
  vt = j / wb;
  mt = b0 + j - (j / wb) * wb;
}

struct HeadTileArgs {
  const bf16 *w;   // [V, dm]
  const bf16 *hp;  // [n, dm]
  int n, V, dm;
  const int32_t *scored_row;  // [n] target row of each scored entry
  const int32_t *tokens;      // [T] token ids of the packed rows
  float *part_m, *part_s;     // forward: [nvt, n] per-tile max and sum
  const float *lse, *dlogp;   // backward: [n]
  bf16 *g;                    // backward: [n, V]
};

// Direct global->LDS copies of the two 256 x 64 tiles of one contraction
// block.  Instruction i (= 4 k + wave) of a tile moves rows 8 i .. 8 i + 7;
// lane L writes LDS bytes 16 L of that 1 KB block, i.e. row 8 i + L / 8 at
// chunk position L % 8, and so fetches the chunk that the swizzle puts there.
// Rows past the last one are clamped to it (finite values that the epilogue
// masks).  In a contraction block that reaches past d_model, chunks past it
// are fetched from chunk 0 of the block instead (in bounds; the fragments
// they feed are zeroed before use).
struct HeadCopy {
  uint32_t off[16];  // byte offset of the lane's chunk in block 0: W rows (k < 8), H_pred rows
  int chunk;         // lane's source chunk in the block

  // (row % 16 = 8 (wave % 2) + lane / 8 for every k, so the chunk is one per lane)
  __device__ __forceinline__ void init(int v0, int m0, int V, int n, int dm, int wave, int lane) {
    chunk = (lane & 7) ^ hswz(8 * wave + (lane >> 3));
    const uint32_t rb = (uint32_t)dm * 2u;  // bytes per row (the host keeps V dm 2, n dm 2 < 2^32)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = (k * HWAVES + wave) * 8 + (lane >> 3);
      off[k] = (uint32_t)min(v0 + row, V - 1) * rb + (uint32_t)(chunk * 16);
      off[8 + k] = (uint32_t)min(m0 + row, n - 1) * rb + (uint32_t)(chunk * 16);
    }
  }

  // Addresses of contraction block kb into the buffers at LDS byte addresses
  // lw / lh.  Scalar 64-bit bases: uniform_ptr zero-extends the low word
  // (readfirstlane returns int; a sign-extended low word would corrupt the
  // high one).  In a block that d_model cuts, a chunk at or past d_model
  // reads chunk 0 of the block instead.
  struct Block {
    uint64_t sw, sh;
    uint32_t fix, lw, lh;
  };
  __device__ __forceinline__ Block block(const bf16 *w, const bf16 *hp, int kb, int dm,
                                         uint32_t lw, uint32_t lh) const {
    Block b;
    b.sw = (uint64_t)(uintptr_t)uniform_ptr(w + (size_t)kb * HK);
    b.sh = (uint64_t)(uintptr_t)uniform_ptr(hp + (size_t)kb * HK);
    b.fix = kb * HK + chunk * 8 >= dm ? (uint32_t)(chunk * 16) : 0u;
    b.lw = lw;
    b.lh = lh;
    return b;
  }

  // copy instruction k (0..15) of a block: 1 KB of W (k < 8) or of H_pred
  template <int k>
  __device__ __forceinline__ void one(const Block &b, int wave) const {
    const uint32_t a = (k < 8 ? b.lw : b.lh) + (uint32_t)(((k & 7) * HWAVES + wave) * 1024);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(a),
                 "v"(off[k] - b.fix), "s"(k < 8 ? b.sw : b.sh)
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
__global__ __launch_bounds__(HWAVES * 64) void head_tile_kernel(HeadTileArgs p, int nvt,
                                                                 int nmt) {
  __shared__ __attribute__((aligned(16))) bf16 sW[2 * HT * HK];
  __shared__ __attribute__((aligned(16))) bf16 sH[2 * HT * HK];
  __shared__ float red_m[2][HT], red_s[2][HT];

  int vt, mt;
  head_tile_of(blockIdx.x, nvt * nmt, nvt, nmt, vt, mt);
  const int v0 = vt * HT, m0 = mt * HT;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int l32 = lane & 31, hi = lane >> 5;
  const int wv = wave & 1, wm = wave >> 1;  // vocab half, row half of the tile
  const int dm = p.dm;
  const int nkb = (dm + HK - 1) / HK;  // 64-deep contraction blocks, the last maybe partial
  const bool tail = (dm % HK) != 0;

  HeadCopy cp;
  cp.init(v0, m0, p.V, p.n, dm, wave, lane);
  const uint32_t lw = lds_address(sW), lh = lds_address(sH);
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

  lds_cchar *const tw0 = lds_bytes(sW) + wv * 128 * 128;
  lds_cchar *const th0 = lds_bytes(sH) + wm * 128 * 128;
  struct Frags {
    bf16x8 a[4], b[4];
  };
  // fragment i (0..7: A 0..3, B 0..3) of 16-deep step st of the block in buffer `cur`
  auto frag = [&](uint32_t cur, int st, int i) {
    return lds_frag((i < 4 ? tw0 : th0) + cur + (i & 3) * 32 * 128, foff[st]);
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
  auto step3 = [&](const Frags &f, Frags &g, const HeadCopy::Block &blk, bool cp_ok, bool rd_ok,
                   uint32_t nxt) {
#define PG_HEAD_SLOT(k)                                                                    \
  acc[(k) >> 2][(k) & 3] = mfma32(f.a[(k) >> 2], f.b[(k) & 3], acc[(k) >> 2][(k) & 3]);    \
  if (cp_ok) cp.one<k>(blk, wave);                                                         \
  if (((k) & 1) && rd_ok) {                                                                \
    constexpr int i = (k) >> 1;                                                            \
    if (i < 4)                                                                             \
      g.a[i & 3] = frag(nxt, 0, i);                                                        \
    else                                                                                   \
      g.b[i & 3] = frag(nxt, 0, i);                                                        \
  }
    PG_HEAD_SLOT(0) PG_HEAD_SLOT(1) PG_HEAD_SLOT(2) PG_HEAD_SLOT(3)
    PG_HEAD_SLOT(4) PG_HEAD_SLOT(5) PG_HEAD_SLOT(6) PG_HEAD_SLOT(7)
    PG_HEAD_SLOT(8) PG_HEAD_SLOT(9) PG_HEAD_SLOT(10) PG_HEAD_SLOT(11)
    PG_HEAD_SLOT(12) PG_HEAD_SLOT(13) PG_HEAD_SLOT(14) PG_HEAD_SLOT(15)
#undef PG_HEAD_SLOT
  };

  // Whole 64-deep blocks, two in flight: block kb + 2 is copied into the
  // buffer of block kb once every wave holds block kb's last fragments in
  // registers (the barrier between its steps 2 and 3), and block kb + 1's
  // first fragments are read while step 3 of block kb multiplies.
  const int nfull = dm / HK;
  cp.all(cp.block(p.w, p.hp, 0, dm, lw, lh), wave);
  if (nkb > 1) {
    cp.all(cp.block(p.w, p.hp, 1, dm, lw + BUF, lh + BUF), wave);
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
    step3(f1, f0, cp.block(p.w, p.hp, kb + 2, dm, lw + cur, lh + cur), kb + 2 < nkb,
          kb + 1 < nfull, nxt);
  }
  if (tail) {
    // the last, partial block (in LDS since the last barrier): steps past
    // d_model are skipped, and in a step that d_model splits
    // (d_model % 16 == 8) the upper lane half's 8 contraction values, which
    // lie past it, are zeroed in both operands
    const uint32_t cur = (nfull & 1) * BUF;
    const int rest = dm - nfull * HK;  // 8 .. 56
    for (int st = 0; st < 4; ++st) {
      if (16 * st >= rest) break;
      Frags f;
      load(f, cur, st);
      if (16 * st + 8 * hi >= rest) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f.a[i] = bf16x8{};
          f.b[i] = bf16x8{};
        }
      }
      mma(f);
    }
  }

  // vocab entry of register r of block a in this lane: vb + 32 a + mfma_row(r, hi)
  const int vb = v0 + wv * 128;
  if constexpr (EPI == 0) {
    // per scored row of the wave: max and sum of exp(z - max) over its 128
    // vocab entries (64 in the lane, 64 in its partner in the other half of
    // the wave); with kMask, entries past the vocabulary (the last vocab
    // tile) take no part, and a slab wholly past it gives max -inf, sum 0
    auto rows = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
      auto val = [&](int a, int b, int r) {
        const float z = acc[a][b][r];
        if constexpr (kMask) return vb + 32 * a + mfma_row(r, hi) < p.V ? z : -INFINITY;
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
        const int rl = wm * 128 + b * 32 + l32;  // row inside the tile
        if (hi == 0) {
          red_m[wv][rl] = mx;
          red_s[wv][rl] = sum;
        }
      }
    };
    if (v0 + HT <= p.V)
      rows(std::false_type{});
    else
      rows(std::true_type{});
    __syncthreads();
    // the two vocab halves of each row, in order
    for (int rl = threadIdx.x; rl < HT; rl += HWAVES * 64) {
      const int row = m0 + rl;
      if (row >= p.n) continue;
      const float ma = red_m[0][rl], mb = red_m[1][rl];
      const float m = fmaxf(ma, mb);
      const float sum = red_s[0][rl] * fast_exp2((ma - m) * kLog2e) +
                        red_s[1][rl] * fast_exp2((mb - m) * kLog2e);
      p.part_m[(size_t)vt * p.n + row] = m;
      p.part_s[(size_t)vt * p.n + row] = sum;
    }
  } else {
    const bool vfull = v0 + HT <= p.V;
    const bool vec = (p.V & 3) == 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = m0 + wm * 128 + b * 32 + l32;
      if (row >= p.n) continue;
      const int tok = p.tokens[p.scored_row[row]];
      const float ll = p.lse[row] * kLog2e, d = p.dlogp[row];
      bf16 *grow = p.g + (size_t)row * p.V;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // registers 4 q .. 4 q + 3: vocab entries vq .. vq + 3
          const int vq = vb + 32 * a + 8 * q + 4 * hi;
          float gv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            gv[j] = -d * fast_exp2(fmaf(acc[a][b][4 * q + j], kLog2e, -ll));
          const unsigned o = (unsigned)(tok - vq);
          if (o < 4u) {  // the token's entry: d (1 - e)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (o == (unsigned)j) gv[j] += d;
          }
          if (vec && (vfull || vq < p.V)) {
            *reinterpret_cast<u32x2 *>(grow + vq) = pack4_bf16(gv[0], gv[1], gv[2], gv[3]);
          } else if (!vec) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (vq + j < p.V) grow[vq + j] = (__bf16)gv[j];
          }
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

HeadTileArgs tile_args(const void *hp, const void *w, int n, int V, int dm,
                       const int32_t *scored_row, const int32_t *tokens) {
  HeadTileArgs a{};
  a.w = (const bf16 *)w;
  a.hp = (const bf16 *)hp;
  a.n = n;
  a.V = V;
  a.dm = dm;
  a.scored_row = scored_row;
  a.tokens = tokens;
  return a;
}

}  // namespace

int head_vocab_tiles(int V) { return (V + HT - 1) / HT; }

hipError_t launch_head_logprob(const void *hp, const void *w, const int32_t *scored_row,
                               const int32_t *tokens, float *part_m, float *part_s, float *logp,
                               float *lse, int n, int V, int dm, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int nvt = head_vocab_tiles(V), nmt = (n + HT - 1) / HT;
  HeadTileArgs a = tile_args(hp, w, n, V, dm, scored_row, tokens);
  a.part_m = part_m;
  a.part_s = part_s;
  hipLaunchKernelGGL(head_tile_kernel<0>, dim3(nvt * nmt), dim3(HWAVES * 64), 0, s, a, nvt, nmt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_lse_combine_kernel, dim3((n + 3) / 4), dim3(256), 0, s, part_m, part_s,
                     (const bf16 *)hp, (const bf16 *)w, scored_row, tokens, logp, lse, n, V, dm,
                     nvt);
  return hipGetLastError();
}

hipError_t launch_head_grad(const void *hp, const void *w, const int32_t *scored_row,
                            const int32_t *tokens, const float *lse, const float *dlogp, void *g,
                            int n, int V, int dm, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int nvt = head_vocab_tiles(V), nmt = (n + HT - 1) / HT;
  HeadTileArgs a = tile_args(hp, w, n, V, dm, scored_row, tokens);
  a.lse = lse;
  a.dlogp = dlogp;
  a.g = (bf16 *)g;
  hipLaunchKernelGGL(head_tile_kernel<1>, dim3(nvt * nmt), dim3(HWAVES * 64), 0, s, a, nvt, nmt);
  return hipGetLastError();
}

}  // namespace pg
