// Fused BinaryAttention forward for gfx950 (CDNA4).
//
// Computes, per (b, h) and query i,
//   O_i = sum_j softmax_j(S_ij) V_j,
//   S_ij = scale * alpha_q,i * alpha_k,j * D_ij + bias(h, i, j),
//   D_ij = <sign q_i, sign k_j>
// i.e. the scaled 1-bit QK similarity plus the learnable bias of the
// BinaryAttention summaries ("Representaciones Binarias Escaladas", "Mejora
// mediante Sesgo"), inside one FlashAttention2-style tiled kernel
// ("Implementacion en Hardware").  The pages' kernel ran QK on 1-bit tensor
// cores and P.V in INT8 on an A100; here P.V is bf16 and both products are
// on CDNA4 matrix cores:
//
//   QK  : +/-1 fp4 operands on v_mfma_scale_f32_32x32x64_f8f6f4, the exact
//         integer D in fp32 (one instruction per 64 channels).
//   P.V : O^T += V^T P^T on v_mfma_f32_32x32x16_bf16.  The 32x32 QK result
//         already holds, per lane, one query and 8 keys of each 16-key step,
//         which is the B-operand layout, so P never leaves registers.  The
//         O^T accumulator keeps one query per lane, so the softmax scalars
//         are per lane.  V^T carries rows of ones, so the same product
//         also yields the row sums l (when d % 32 == 0 they are added on the
//         vector ALU instead).
//
// Workgroup: 4 waves x 32 queries = 128 queries of one (b, h).  Each wave
// packs its own 32 queries (signs and alpha_q) from bf16 at the start.  Key
// tiles of 64 live in two LDS buffers: while tile t is computed from one, the
// next tile's fp4 key operands (written by the prologue), key scales, V^T and
// bias window stream into the other with buffer-to-LDS copies.  One barrier
// per tile.  Every LDS address is a per-lane base fixed at kernel start plus
// a constant or a wave-uniform offset; no division runs inside the key loop.
//
// Softmax, in base 2.  Every logit of a workgroup obeys |s| <= M with
//   M = scale log2e max_i alpha_q,i max_j alpha_k,j d + log2e max|b|
// (|D| <= d).  When M <= kFastMaxLogit, exp2(s) lies in [2^-M, 2^M] and
// softmax is taken without any offset (it does not depend on one): one
// multiply, one FMA and one exp2 per score, no running maximum.  Otherwise
// the exact online softmax runs (running row max, rescale skipped while the
// max grows by <= 8, so P <= 2^8).
#include "ba_internal.h"

namespace ba {

// Largest logit bound (log2 units) for the offset-free path: exp2 stays in
// [2^-32, 2^32], row sums below 2^48, so nothing under- or overflows for
// |V| < 2^80.
constexpr float kFastMaxLogit = 32.0f;

// Bias storage per tile buffer, by bias mode (modes that do not use an
// array keep a token 16 bytes of it).
template <int BIAS>
struct BiasSizes {
  static constexpr int kWin =
      BIAS == kBiasRows ? kMaxWindowFloats : (BIAS == kBiasDense ? kDenseTileFloats : 4);
  static constexpr int kGk = BIAS == kBiasTable ? kBN : 4;
};

// One LDS tile buffer.  The kernel declares two of them as separate LDS
// objects, so the compiler can tell the asynchronous copies into one buffer
// from the reads of the other and need not wait for the copies early.
template <int NCH, int CB, int BIAS>
struct TileBuf {
  v4i k[NCH * kBN * 2];                // fp4 key operands [c][key][h]
  float ak[kBN];                        // key scales
  int gk[BiasSizes<BIAS>::kGk];         // grid offsets (table mode)
  uint16_t vt[32 * CB * kBN];           // V^T tile: rows of 64 keys, swizzled
  float win[BiasSizes<BIAS>::kWin];     // bias window (table-row mode) or
                                        // dense bias tile (dense mode)
};

// The row sums l of P: when d % 32 != 0, V^T carries rows of ones (rows d
// and d+4), so accumulator row d of the P.V product holds sum_j P_ij.  When
// d % 32 == 0 (XONES), both passes add the bf16 P pairs on the vector ALU
// into two partial sums per lane, rs[0..1]; at the end of the pass rs[0]
// holds sum_j P_ij in both lanes of the query.
template <int CB, bool XONES>
struct Acc {
  v16f o[CB];
  float rs[2];  // used when XONES
};

// Per-lane and per-workgroup constants.
template <int NCH>
struct Ctx {
  const FwdArgs* a;
  float* table;        // dynamic LDS: the whole bias table (table mode)
  int tid, lane, wave, li, lh;
  int bh, head, q0, qi;
  int64_t tokbase;
  float aq;            // alpha_q * scale * log2e
  float alpha;         // alpha_q itself (the backward's row tokens)
  v4i qop[NCH];        // this lane's query operand (fp4 +/-1)
  // LDS byte offsets inside a TileBuf, per lane
  // off_akb: the key scale this lane holds for the row broadcasts;
  // off_gk: this lane's first grid offset (table mode)
  int off_k, off_akb, off_gk, off_v[4], off_win;
  int yq, xq, yq_lo, fidx;
  // Asynchronous tile copies: wave-uniform bases (scalar registers) plus
  // per-lane 32-bit byte offsets.
  rsrc_t vrs;          // V^T tiles of this (b, h)
  rsrc_t krs;          // fp4 key operand tiles of this (b, h)
  rsrc_t ars;          // key scales of this (b, h)
  rsrc_t brs;          // bias rows of this head (table-row mode)
  int win_bytes;       // bytes of the per-tile bias window (table-row mode)
  rsrc_t drs;          // dense bias of this (b, h) (dense mode)
  uint32_t dvoff;      // this lane's byte offset in its dense-tile copies
  uint32_t dld2;       // dense bias row stride in bytes
  int off_dn[4];       // this lane's dense-tile LDS bytes, group b of block 0
  int off8[2];         // this lane's int8 value-operand LDS bytes, per block (8-bit P.V)
};

// Uniform per-tile position of the keys on the grid (table-row mode).
struct KeyPos {
  int k0;
  int ky[2], kx[2];  // row and column of the first key of each 32-key block
};

__device__ __forceinline__ KeyPos next_keys(const KeyPos& p, int gw) {
  KeyPos n;
  n.k0 = p.k0 + kBN;
  // Blocks are 32-aligned and gw % 32 == 0: a block never straddles rows.
  // The wrap flag is formed with a shift, which keeps it in scalar registers.
  int x = p.kx[1] + 32, w = static_cast<int>(static_cast<uint32_t>(gw - 1 - x) >> 31);
  n.ky[0] = p.ky[1] + w;
  n.kx[0] = x - w * gw;
  x = n.kx[0] + 32;
  w = static_cast<int>(static_cast<uint32_t>(gw - 1 - x) >> 31);
  n.ky[1] = n.ky[0] + w;
  n.kx[1] = x - w * gw;
  return n;
}

// Floats of the workgroup reductions' LDS scratch (three per wave).
constexpr int kRedFloats = 3 * kThreads / 64;

// The workgroup maxima of three values with one pair of barriers.
__device__ __forceinline__ v3f block_max3(float x, float y, float z, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    x = fmaxf(x, __shfl_xor(x, off, 64));
    y = fmaxf(y, __shfl_xor(y, off, 64));
    z = fmaxf(z, __shfl_xor(z, off, 64));
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[3 * (threadIdx.x >> 6)] = x;
    red[3 * (threadIdx.x >> 6) + 1] = y;
    red[3 * (threadIdx.x >> 6) + 2] = z;
  }
  __syncthreads();
  v3f r = {red[0], red[1], red[2]};
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w)
    r = v3f{fmaxf(r[0], red[3 * w]), fmaxf(r[1], red[3 * w + 1]), fmaxf(r[2], red[3 * w + 2])};
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r += red[w];
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

// LDS loads use whole vector types (ext_vector_type), never the HIP float4 /
// int4 structs: a struct load is split into scalar loads, which the backend
// re-merges without the alias scope that tells the compiler the load cannot
// touch the other tile buffer, and it then waits for every copy in flight
// before the load.
template <typename T>
__device__ __forceinline__ T lds_load(const void* base, int byte_off) {
  return *reinterpret_cast<const T*>(__builtin_assume_aligned(static_cast<const char*>(base) + byte_off, 16));
}

// ---------------------------------------------------------------- staging --
// Starts the copies of key tile `t` (first key kp.k0) into `tb`: the fp4 key
// operands, V^T, key scales and (table-row mode) the bias window go straight
// to LDS (buffer_load ... lds: lane l of a wave fills bytes [16l, 16l+16) of
// a 1 KiB block, or [4l, 4l+4) of a 256-byte block).  In table mode the
// grid offsets of the tile's keys are computed and stored directly: `tb` was
// last read before the previous barrier.
// What a tile copy brings of the values: nothing (the 8-bit path's row
// maximum pass), the bf16 V^T tile, or the int8 value-code tile.
enum VCopy { kVNone = 0, kVBf16 = 1, kVInt8 = 2 };

// TB is TileBuf<NCH, CB, BIAS> or the backward's tile buffer (same members).
template <int NCH, int CB, int BIAS, int VM = kVBf16, class TB = TileBuf<NCH, CB, BIAS>>
__device__ __forceinline__ void copy_tile_async(const Ctx<NCH>& c, TB& tb, int t, const KeyPos& kp) {
  const FwdArgs& a = *c.a;
  constexpr int kKBytes = NCH * kBN * 2 * 16;
  char* kdst = reinterpret_cast<char*>(&tb.k[0]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (c.wave + 4 * j < kKBytes / 1024)
      dma16(c.krs, kdst + (c.wave + 4 * j) * 1024, static_cast<uint32_t>(c.lane * 16),
            static_cast<uint32_t>(t * kKBytes + (c.wave + 4 * j) * 1024));
  constexpr int kVtBytes = 32 * CB * kBN * 2;
  char* vdst = reinterpret_cast<char*>(&tb.vt[0]);
  // this lane's byte in its 1 KiB pieces, recomputed here rather than kept
  // in a register through the key loop
  const uint32_t loff = static_cast<uint32_t>(c.wave * 1024 + c.lane * 16);
  if (VM == kVBf16) {
#pragma unroll
    for (int j = 0; j < kVtBytes / 4096; ++j)
      dma16(c.vrs, vdst + (c.wave + 4 * j) * 1024, loff, static_cast<uint32_t>(t * kVtBytes + j * 4096));
  } else if (VM == kVInt8) {
    // 2 CB pieces of 1 KiB (dpad rows of 64 bytes), piece = wave + 4 j
    constexpr int kV8Bytes = 32 * CB * kBN;
#pragma unroll
    for (int j = 0; j < (2 * CB + 3) / 4; ++j)
      if (c.wave + 4 * j < 2 * CB)
        dma16(c.vrs, vdst + (c.wave + 4 * j) * 1024, static_cast<uint32_t>(c.lane * 16),
              static_cast<uint32_t>(t * kV8Bytes + (c.wave + 4 * j) * 1024));
  }
  if (c.wave == 0) dma4(c.ars, &tb.ak[0], static_cast<uint32_t>(c.lane * 4), static_cast<uint32_t>(kp.k0 * 4));
  if (BIAS == kBiasRows) {
    // window rows start at dy = yq_lo - yk_hi; yk_hi is the row of block 1
    const int dy0 = c.yq_lo - kp.ky[1] + a.gh - 1 + kBiasPadRows;
    const uint32_t bs = static_cast<uint32_t>(dy0 * 16 * a.Lpad);
    char* bdst = reinterpret_cast<char*>(&tb.win[0]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (static_cast<int>(loff) + 4096 * j < c.win_bytes)
        dma16(c.brs, bdst + (c.wave + 4 * j) * 1024, loff + 4096 * j, bs);
  }
  if (BIAS == kBiasDense) {
    // 128 query rows x 64 keys of bf16 = 16 pieces of 1 KiB, 4 per wave.
    // Piece m holds rows 8m .. 8m+7; lane l fills slot 64m + l, i.e. row
    // 8m + l/8 and 16-byte chunk (l%8) ^ ((l/16) & 3) of that row (the XOR
    // spreads the rows a wave reads over the LDS banks).
    char* ddst = reinterpret_cast<char*>(&tb.win[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = c.wave + 4 * j;
      dma16_nt(c.drs, ddst + m * 1024, c.dvoff + static_cast<uint32_t>(m * 8) * c.dld2 + static_cast<uint32_t>(kp.k0 * 2),
               0u);
    }
  }
  if (BIAS == kBiasTable && c.tid < kBN) {
    const int j = (kp.k0 + c.tid < a.N) ? kp.k0 + c.tid : a.N - 1;
    const int yj = j / a.gw;
    tb.gk[c.tid] = yj * (2 * a.gw - 1) + (j - yj * a.gw);
  }
}

// ---------------------------------------------------------------- compute --
// Byte offset of this lane's bias entries for block `blk` inside the tile's
// window.  The empty asm makes it one opaque value, so every window read is a
// single constant offset from it; a longer chain of address arithmetic hides
// from the compiler which LDS buffer the read touches, and it then waits for
// the copies into the other buffer before the read.
template <int NCH>
__device__ __forceinline__ int window_offset(const Ctx<NCH>& c, const KeyPos& kp, int blk) {
  int off = c.off_win + (kp.ky[1] - kp.ky[blk]) * 16 * c.a->Lpad + kp.kx[blk] * 4;
  asm("" : "+v"(off));
  return off;
}

// Logits of one 32-key block in base 2:
//   D * alpha_k * (alpha_q scale log2e) + log2e b
template <bool MASK, int NCH, int CB, int BIAS, class TB = TileBuf<NCH, CB, BIAS>>
__device__ __forceinline__ void block_logits(const Ctx<NCH>& c, const TB& tb, const KeyPos& kp,
                                             int blk, const v16f& s, float (&sc)[16]) {
  const FwdArgs& a = *c.a;
  int woff = 0;
  if (BIAS == kBiasRows) woff = window_offset(c, kp, blk);
  const float akv = lds_load<float>(tb.ak, c.off_akb + blk * 128);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float u0 = s[4 * b] * row_bcast(akv, 4 * b), u1 = s[4 * b + 1] * row_bcast(akv, 4 * b + 1);
    const float u2 = s[4 * b + 2] * row_bcast(akv, 4 * b + 2), u3 = s[4 * b + 3] * row_bcast(akv, 4 * b + 3);
    if (BIAS == kBiasRows) {
      const v4f bias = lds_load<v4f>(tb.win, woff + 32 * b);
      sc[4 * b + 0] = fmaf(u0, c.aq, bias.x);
      sc[4 * b + 1] = fmaf(u1, c.aq, bias.y);
      sc[4 * b + 2] = fmaf(u2, c.aq, bias.z);
      sc[4 * b + 3] = fmaf(u3, c.aq, bias.w);
    } else if (BIAS == kBiasTable) {
      const v4i g = lds_load<v4i>(tb.gk, c.off_gk + (blk * 32 + 8 * b) * 4);
      sc[4 * b + 0] = fmaf(u0, c.aq, c.table[c.fidx - g.x]);
      sc[4 * b + 1] = fmaf(u1, c.aq, c.table[c.fidx - g.y]);
      sc[4 * b + 2] = fmaf(u2, c.aq, c.table[c.fidx - g.z]);
      sc[4 * b + 3] = fmaf(u3, c.aq, c.table[c.fidx - g.w]);
    } else if (BIAS == kBiasDense) {
      // keys 4 lh .. 4 lh + 3 of group b: four bf16 in two dwords; natural
      // units (c.aq holds alpha_q * scale), log2e comes with the row shift
      const v2u w = lds_load<v2u>(tb.win, c.off_dn[b] + 64 * blk);
      sc[4 * b + 0] = fmaf(u0, c.aq, __uint_as_float(w.x << 16));
      sc[4 * b + 1] = fmaf(u1, c.aq, __uint_as_float(w.x & 0xffff0000u));
      sc[4 * b + 2] = fmaf(u2, c.aq, __uint_as_float(w.y << 16));
      sc[4 * b + 3] = fmaf(u3, c.aq, __uint_as_float(w.y & 0xffff0000u));
    } else {
      sc[4 * b + 0] = u0 * c.aq;
      sc[4 * b + 1] = u1 * c.aq;
      sc[4 * b + 2] = u2 * c.aq;
      sc[4 * b + 3] = u3 * c.aq;
    }
  }
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kp.k0 + blk * 32 + 8 * (r >> 2) + 4 * c.lh + (r & 3);
      if (key >= a.N) sc[r] = -INFINITY;
    }
  }
}

// Exact path only: running row max over this block (mrow, in log2 units);
// rescales the accumulators when it grows by more than 8, and shifts the
// logits by it.  NATURAL: the logits come in natural-log units and are
// turned into log2 units by the shift itself (one FMA per logit).  A row
// whose keys so far all have logit -inf (a dense bias or a table may mask
// keys) keeps mrow = -inf, its (zero) sums unscaled, and is shifted by 0, so
// its probabilities stay 0, not NaN.
template <bool NATURAL, int CB, bool XONES>
__device__ __forceinline__ void block_rescale(float (&sc)[16], Acc<CB, XONES>& acc, float& mrow) {
  float mt = sc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
  mt = max_halves(mt);
  if (NATURAL) mt *= kLog2e;
  const float mnew = fmaxf(mrow, mt);
  if (__any(mnew > mrow + 8.0f)) {
    const float f = mnew > -INFINITY ? fast_exp2(mrow - mnew) : 1.0f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc.o[cb] *= f;
    if (XONES) {
      acc.rs[0] *= f;
      acc.rs[1] *= f;
    }
    mrow = mnew;
  }
  if (NATURAL) {
    const float shift = mrow == -INFINITY ? 0.0f : mrow;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = fmaf(sc[r], kLog2e, -shift);
  } else {
    const float shift = mrow == -INFINITY ? 0.0f : mrow;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] -= shift;
  }
}

// ------------------------------------------------- pipelined fast path ----
// P.V of a finished 32-key block waits in registers (bf16 P and its V^T
// operands) and is issued right after the next block's QK, so its matrix
// instructions run while that block's logits are formed: the matrix cores
// and the vector ALUs of a SIMD overlap even within one wave, and the V^T
// operands no longer tie the block to its LDS buffer (the pipeline runs
// across tile barriers).  Issuing them all at once frees their registers
// before the logits are live; spreading them over the four groups of keys
// measured no faster.
template <int CB>
struct PendingPV {
  uint32_t pk[8];     // bf16 P, 16 keys x 2 steps
  v8bf vop[2][CB];    // V^T operands of the two 16-key steps
};

template <int CB, bool XONES>
__device__ __forceinline__ void pv_mfma(int i, const PendingPV<CB>& pp, Acc<CB, XONES>& acc) {
  const int half = i / CB, cb = i % CB;
  const v4u pw = {pp.pk[4 * half], pp.pk[4 * half + 1], pp.pk[4 * half + 2], pp.pk[4 * half + 3]};
  acc.o[cb] = mfma_bf16_32x32x16(pp.vop[half][cb], __builtin_bit_cast(v8bf, pw), acc.o[cb]);
}

// Block `blk` of tile `tb`: its QK, the pending block's P.V, then this
// block's logits / exp2 / bf16 packing; this block becomes pending.
template <bool MASK, bool HAVE_PENDING, int NCH, int CB, bool XONES, int BIAS>
__device__ __forceinline__ void pipelined_block(const Ctx<NCH>& c, const TileBuf<NCH, CB, BIAS>& tb, const KeyPos& kp,
                                                int blk, PendingPV<CB>& pp, Acc<CB, XONES>& acc) {
  const FwdArgs& a = *c.a;
  constexpr int kMf = 2 * CB;
  v16f s = v16f{};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
    s = mfma_signs_32x32x64(lds_load<v4i>(tb.k, c.off_k + ch * 2048 + blk * 1024), c.qop[ch], s);
  if (HAVE_PENDING) {
#pragma unroll
    for (int i = 0; i < kMf; ++i) pv_mfma<CB, XONES>(i, pp, acc);
  }
  int woff = 0;
  if (BIAS == kBiasRows) woff = window_offset(c, kp, blk);
  const float akv = lds_load<float>(tb.ak, c.off_akb + blk * 128);
  uint32_t pk[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float x0 = s[4 * b] * row_bcast(akv, 4 * b), x1 = s[4 * b + 1] * row_bcast(akv, 4 * b + 1);
    float x2 = s[4 * b + 2] * row_bcast(akv, 4 * b + 2), x3 = s[4 * b + 3] * row_bcast(akv, 4 * b + 3);
    if (BIAS == kBiasRows) {
      const v4f bias = lds_load<v4f>(tb.win, woff + 32 * b);
      x0 = fmaf(x0, c.aq, bias.x);
      x1 = fmaf(x1, c.aq, bias.y);
      x2 = fmaf(x2, c.aq, bias.z);
      x3 = fmaf(x3, c.aq, bias.w);
    } else if (BIAS == kBiasTable) {
      const v4i g = lds_load<v4i>(tb.gk, c.off_gk + (blk * 32 + 8 * b) * 4);
      x0 = fmaf(x0, c.aq, c.table[c.fidx - g.x]);
      x1 = fmaf(x1, c.aq, c.table[c.fidx - g.y]);
      x2 = fmaf(x2, c.aq, c.table[c.fidx - g.z]);
      x3 = fmaf(x3, c.aq, c.table[c.fidx - g.w]);
    } else {
      x0 *= c.aq;
      x1 *= c.aq;
      x2 *= c.aq;
      x3 *= c.aq;
    }
    if (MASK) {
      const int key = kp.k0 + blk * 32 + 8 * b + 4 * c.lh;
      if (key + 0 >= a.N) x0 = -INFINITY;
      if (key + 1 >= a.N) x1 = -INFINITY;
      if (key + 2 >= a.N) x2 = -INFINITY;
      if (key + 3 >= a.N) x3 = -INFINITY;
    }
    pk[2 * b] = pack_bf16x2(fast_exp2(x0), fast_exp2(x1));
    pk[2 * b + 1] = pack_bf16x2(fast_exp2(x2), fast_exp2(x3));
    // Row sums on the vector ALU (two partial sums per lane), cheaper here
    // than the extra matrix instructions of a ones block; they add the same
    // bf16 P that multiplies V.
    if (XONES) acc.rs[b & 1] = add_bf16x2(pk[2 * b], add_bf16x2(pk[2 * b + 1], acc.rs[b & 1]));
  }
  // this block becomes pending: P and its V^T operands
#pragma unroll
  for (int j = 0; j < 8; ++j) pp.pk[j] = pk[j];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      pp.vop[half][cb] = lds_load<v8bf>(tb.vt, c.off_v[2 * blk + half] + cb * 4096);
}

// Wave priority for key tile t of nkt: 3 (the highest) through the first
// five eighths of the keys, then 2, 1 and 0 for the last three.  The waves of
// a SIMD come from several workgroups, and when they are equal the hardware
// favours the oldest, so the first workgroup of a CU would finish long before
// the last, which then runs alone with one wave per SIMD and no second wave to
// overlap its matrix and vector work with.  Lowering a wave's priority as it
// nears the end lets the later workgroups catch up.  Only for grids whose
// workgroups are all resident at once (the host sets prio_balance): with
// more workgroups than slots, holding back the ones about to finish delays
// the slots the rest are waiting for.
__device__ __forceinline__ void tile_priority(const FwdArgs& a, int t, int nkt) {
  if (!a.prio_balance) return;
  const int e = (8 * t) / nkt;
  if (e <= 4)
    __builtin_amdgcn_s_setprio(3);
  else if (e == 5)
    __builtin_amdgcn_s_setprio(2);
  else if (e == 6)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Pipelined (offset-free) version of pass_step: tile t's two blocks each
// overlap the previous block's P.V.
template <bool FIRST, int NCH, int CB, bool XONES, int BIAS>
__device__ __forceinline__ void fast_step(const Ctx<NCH>& c, const TileBuf<NCH, CB, BIAS>& cur, TileBuf<NCH, CB, BIAS>& nxt,
                                          int t, int nkt, KeyPos& kp, Acc<CB, XONES>& acc, PendingPV<CB>& pp) {
  const FwdArgs& a = *c.a;
  const bool more = t + 1 < nkt;
  const KeyPos kn = next_keys(kp, a.gw);
  if (more) copy_tile_async<NCH, CB, BIAS>(c, nxt, t + 1, kn);
  if (BIAS == kBiasRows) {
    // N % 32 == 0 here: a ragged last tile is one real block and one block
    // of padded keys, which is skipped (see pass_step)
    pipelined_block<false, !FIRST, NCH, CB, XONES, BIAS>(c, cur, kp, 0, pp, acc);
    if (kp.k0 + 32 < a.N) pipelined_block<false, true, NCH, CB, XONES, BIAS>(c, cur, kp, 1, pp, acc);
  } else if (kp.k0 + kBN <= a.N) {  // a full tile; the ragged last one is masked
    pipelined_block<false, !FIRST, NCH, CB, XONES, BIAS>(c, cur, kp, 0, pp, acc);
    pipelined_block<false, true, NCH, CB, XONES, BIAS>(c, cur, kp, 1, pp, acc);
  } else {
    pipelined_block<true, !FIRST, NCH, CB, XONES, BIAS>(c, cur, kp, 0, pp, acc);
    pipelined_block<true, true, NCH, CB, XONES, BIAS>(c, cur, kp, 1, pp, acc);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  kp = kn;
}

template <int NCH, int CB, bool XONES, int BIAS>
__device__ __forceinline__ void run_fast_pass(const Ctx<NCH>& c, TileBuf<NCH, CB, BIAS>& tb0, TileBuf<NCH, CB, BIAS>& tb1,
                                              Acc<CB, XONES>& acc) {
  const FwdArgs& a = *c.a;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc.o[cb] = v16f{};
  acc.rs[0] = acc.rs[1] = 0.0f;
  KeyPos kp;
  kp.k0 = 0;
  kp.ky[0] = 0;
  kp.kx[0] = 0;
  kp.ky[1] = (BIAS == kBiasRows && a.gw == 32) ? 1 : 0;
  kp.kx[1] = (BIAS == kBiasRows && a.gw == 32) ? 0 : 32;
  copy_tile_async<NCH, CB, BIAS>(c, tb0, 0, kp);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nkt = (a.N + kBN - 1) / kBN;
  PendingPV<CB> pp;
  fast_step<true, NCH, CB, XONES, BIAS>(c, tb0, tb1, 0, nkt, kp, acc, pp);
  for (int t = 1; t < nkt; t += 2) {
    tile_priority(a, t, nkt);
    fast_step<false, NCH, CB, XONES, BIAS>(c, tb1, tb0, t, nkt, kp, acc, pp);
    if (t + 1 < nkt) fast_step<false, NCH, CB, XONES, BIAS>(c, tb0, tb1, t + 1, nkt, kp, acc, pp);
  }
  // drain: the last block's P.V
#pragma unroll
  for (int i = 0; i < 2 * CB; ++i) pv_mfma<CB, XONES>(i, pp, acc);
  // the row sums, in the register the epilogue reads: both halves of each
  // query's keys (lanes l and l^32)
  if (XONES) acc.rs[0] = sum_halves(acc.rs[0] + acc.rs[1]);
}

// ------------------------------------------------ pipelined exact path ----
// The online softmax with a running row maximum (exact path), pipelined as
// the fast path is: the pending block's P.V is issued after this block's QK,
// before this block's maximum is known, so a rescale of the accumulators
// also covers the pending product.
template <bool MASK, bool HAVE_PENDING, int NCH, int CB, bool XONES, int BIAS>
__device__ __forceinline__ void exact_block(const Ctx<NCH>& c, const TileBuf<NCH, CB, BIAS>& tb, const KeyPos& kp,
                                            int blk, PendingPV<CB>& pp, Acc<CB, XONES>& acc, float& mrow) {
  v16f s = v16f{};
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
    s = mfma_signs_32x32x64(lds_load<v4i>(tb.k, c.off_k + ch * 2048 + blk * 1024), c.qop[ch], s);
  if (HAVE_PENDING) {
#pragma unroll
    for (int i = 0; i < 2 * CB; ++i) pv_mfma<CB, XONES>(i, pp, acc);
  }
  float sc[16];
  block_logits<MASK, NCH, CB, BIAS>(c, tb, kp, blk, s, sc);
  block_rescale<BIAS == kBiasDense>(sc, acc, mrow);
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pk[j] = pack_bf16x2(fast_exp2(sc[2 * j]), fast_exp2(sc[2 * j + 1]));
  if (XONES) {
#pragma unroll
    for (int b = 0; b < 4; ++b) acc.rs[b & 1] = add_bf16x2(pk[2 * b], add_bf16x2(pk[2 * b + 1], acc.rs[b & 1]));
  }
  // this block becomes pending: P and its V^T operands
#pragma unroll
  for (int j = 0; j < 8; ++j) pp.pk[j] = pk[j];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      pp.vop[half][cb] = lds_load<v8bf>(tb.vt, c.off_v[2 * blk + half] + cb * 4096);
}

// One key tile of the exact path: start the copies of tile t+1 into `nxt`,
// compute tile t from `cur`, wait, barrier.
template <bool FIRST, int NCH, int CB, bool XONES, int BIAS>
__device__ __forceinline__ void exact_step(const Ctx<NCH>& c, const TileBuf<NCH, CB, BIAS>& cur,
                                           TileBuf<NCH, CB, BIAS>& nxt, int t, int nkt, KeyPos& kp,
                                           Acc<CB, XONES>& acc, PendingPV<CB>& pp, float& mrow) {
  const FwdArgs& a = *c.a;
  const bool more = t + 1 < nkt;
  const KeyPos kn = next_keys(kp, a.gw);
  if (more) copy_tile_async<NCH, CB, BIAS>(c, nxt, t + 1, kn);
  // Keys past N must get probability 0 on the ragged last tile.  The
  // padding rows of the table-row bias keep the window reads inside the
  // rows but do not cover every padded key (one on grid row >= gh, seen from
  // a query on grid row >= 1, falls on a real table row).  Table rows have
  // N % 32 == 0, so there the ragged tile is a real block and a block of
  // padded keys, which is skipped; the other modes mask key by key.
  if (BIAS == kBiasRows) {
    exact_block<false, !FIRST, NCH, CB, XONES, BIAS>(c, cur, kp, 0, pp, acc, mrow);
    if (kp.k0 + 32 < a.N) exact_block<false, true, NCH, CB, XONES, BIAS>(c, cur, kp, 1, pp, acc, mrow);
  } else if (kp.k0 + kBN <= a.N) {
    exact_block<false, !FIRST, NCH, CB, XONES, BIAS>(c, cur, kp, 0, pp, acc, mrow);
    exact_block<false, true, NCH, CB, XONES, BIAS>(c, cur, kp, 1, pp, acc, mrow);
  } else {
    exact_block<true, !FIRST, NCH, CB, XONES, BIAS>(c, cur, kp, 0, pp, acc, mrow);
    exact_block<true, true, NCH, CB, XONES, BIAS>(c, cur, kp, 1, pp, acc, mrow);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  kp = kn;
}

// One pass over all keys with the exact softmax; O^T (and the row sums)
// accumulate in acc.  Returns the row maximum (log2 units) the sums are
// taken against.
template <int NCH, int CB, bool XONES, int BIAS>
__device__ __forceinline__ float run_exact_pass(const Ctx<NCH>& c, TileBuf<NCH, CB, BIAS>& tb0,
                                                TileBuf<NCH, CB, BIAS>& tb1, Acc<CB, XONES>& acc) {
  const FwdArgs& a = *c.a;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc.o[cb] = v16f{};
  acc.rs[0] = acc.rs[1] = 0.0f;
  float mrow = -INFINITY;
  KeyPos kp;
  kp.k0 = 0;
  kp.ky[0] = 0;
  kp.kx[0] = 0;
  kp.ky[1] = (BIAS == kBiasRows && a.gw == 32) ? 1 : 0;
  kp.kx[1] = (BIAS == kBiasRows && a.gw == 32) ? 0 : 32;
  copy_tile_async<NCH, CB, BIAS>(c, tb0, 0, kp);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nkt = (a.N + kBN - 1) / kBN;
  PendingPV<CB> pp;
  exact_step<true, NCH, CB, XONES, BIAS>(c, tb0, tb1, 0, nkt, kp, acc, pp, mrow);
  for (int t = 1; t < nkt; t += 2) {
    tile_priority(a, t, nkt);
    exact_step<false, NCH, CB, XONES, BIAS>(c, tb1, tb0, t, nkt, kp, acc, pp, mrow);
    if (t + 1 < nkt) exact_step<false, NCH, CB, XONES, BIAS>(c, tb0, tb1, t + 1, nkt, kp, acc, pp, mrow);
  }
  // drain: the last block's P.V
#pragma unroll
  for (int i = 0; i < 2 * CB; ++i) pv_mfma<CB, XONES>(i, pp, acc);
  if (XONES) acc.rs[0] = sum_halves(acc.rs[0] + acc.rs[1]);
  return mrow;
}

// Everything a workgroup sets up before its key loop: its (b, h) and
// query tile, this lane's packed query, the per-lane LDS offsets, the
// buffer resources of the tile copies, the bias table in LDS (table mode).
// Returns the logit bound M (log2 units) of the workgroup.
// SMALL: the one-launch kernel for short sequences, whose key scales are in
// LDS already; kmax_small is their maximum over the head.
template <int NCH, int CB, int BIAS, bool SMALL = false>
__device__ __forceinline__ float workgroup_setup(Ctx<NCH>& c, const FwdArgs& a, float* red, float* s_table,
                                                 float kmax_small = 0.0f) {
  c.a = &a;
  c.table = s_table;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(c.tid >> 6);
  c.li = c.lane & 31;
  c.lh = c.lane >> 5;

  int wg = blockIdx.x;
  if (a.xcd_remap) {
    const int per = a.nwg >> 3;
    wg = (wg & 7) * per + (wg >> 3);
  }
  int qt;
  if (BIAS == kBiasDense && a.dense_shared) {
    // One bias for the whole batch: the B workgroups that read the same
    // bias tiles get consecutive indices (batch fastest), so they run side
    // by side on one XCD and the second reads of a tile hit its L2.
    const int b = wg % a.B, t = wg / a.B;
    const int h = t / a.nqt;
    qt = t - h * a.nqt;
    c.bh = b * a.H + h;
  } else {
    c.bh = wg / a.nqt;
    qt = wg - c.bh * a.nqt;
  }
  c.head = c.bh % a.H;
  c.q0 = qt * kBM;
  c.qi = c.q0 + c.wave * 32 + c.li;
  c.tokbase = static_cast<int64_t>(c.bh) * a.Npad;

  // ---- this lane's query, packed straight from Q ---------------------------
  // Lane (li, lh) forms the sign words 2 ch + lh of query qi (channels
  // 32 word .. 32 word + 31) and sums |q| over them; the partner lane l ^ 32
  // holds the other words, so the two partial sums make the scale
  // alpha_q = mean |q| ("Representaciones Binarias Escaladas").  Queries past
  // N are all zero: scale 0.
  float qpart = 0.0f;
  {
    const uint16_t* qrow = a.q + token_offset(a.qs, c.bh / a.H, c.head, c.qi < a.N ? c.qi : 0);
    // every piece is loaded before any is used: a load consumed at once
    // waits for the one before it, one memory round trip per piece
    uint4 qv[NCH][4];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c0 = 32 * (2 * ch + c.lh) + 8 * k;
        qv[ch][k] = make_uint4(0u, 0u, 0u, 0u);
        if (c.qi < a.N && c0 < a.d) qv[ch][k] = *reinterpret_cast<const uint4*>(qrow + c0);
      }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int word = 2 * ch + c.lh;
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c0 = 32 * word + 8 * k;
        if (c.qi < a.N && c0 < a.d) {
          float part;
          w |= chunk_signs(qv[ch][k], part) << (8 * k);
          qpart += part;
        }
      }
      c.qop[ch] = expand_signs_fp4(w, fp4_magnitude(word_valid(a.d, word)));
    }
  }
  const float alpha_q = sum_halves(qpart) / static_cast<float>(a.d);
  c.aq = alpha_q * a.qscale;
  c.alpha = alpha_q;

  // ---- per-lane LDS offsets ------------------------------------------------
  c.off_k = (c.li * 2 + c.lh) * 16;
  // Key scales reach the logits by row broadcast: accumulator register r of
  // every lane in a 16-lane row holds key 8(r/4) + 4(lane/32) + r%4 of the
  // block, so lane 16 row + r keeps that key's scale and register r reads it
  // with row_newbcast:r, folded into the multiply.
  c.off_akb = 4 * (8 * ((c.lane & 15) >> 2) + 4 * c.lh + (c.lane & 3));
  c.off_gk = c.lh * 16;
  {
    const int sw = (c.li >> 1) & 7;
#pragma unroll
    for (int p = 0; p < 4; ++p) c.off_v[p] = c.li * 128 + (((2 * p + c.lh) ^ sw) << 4);
  }
  c.yq = c.xq = c.yq_lo = c.fidx = c.off_win = 0;
  if (BIAS == kBiasRows || BIAS == kBiasTable) {
    c.yq = c.qi / a.gw;
    c.xq = c.qi - c.yq * a.gw;
  }
  if (BIAS == kBiasRows) {
    // bias(i, j) = R[dy][gw-1-xi+xj], read from copy s = (gw-1-xi) & 3 at an
    // aligned float offset, in window row (yq - yq_lo) + (yk_hi - yk).
    c.yq_lo = c.q0 / a.gw;
    const int bsel = (a.gw - 1 - c.xq) & 3;
    c.off_win = (((c.yq - c.yq_lo) * 4 + bsel) * a.Lpad + (a.gw - 1 - c.xq + 4 * c.lh - bsel)) * 4;
  }

  // ---- global sources of the tile copies -----------------------------------
  constexpr int kVtBytes = 32 * CB * kBN * 2;
  // Per-head ranges: every byte of a range lies inside the workspace section
  // it names, and each range is far below 2^31 bytes.
  c.vrs = make_rsrc(reinterpret_cast<const char*>(a.vt) + static_cast<int64_t>(c.bh) * (a.Npad / kBN) * kVtBytes,
                    static_cast<uint32_t>((a.Npad / kBN) * kVtBytes));
  constexpr int kKBytes = NCH * kBN * 2 * 16;
  c.krs = make_rsrc(reinterpret_cast<const char*>(a.kop) + static_cast<int64_t>(c.bh) * (a.Npad / kBN) * kKBytes,
                    static_cast<uint32_t>((a.Npad / kBN) * kKBytes));
  c.ars = make_rsrc(a.alpha_k + c.tokbase, static_cast<uint32_t>(a.Npad * 4));
  c.brs = c.ars;
  c.win_bytes = 0;
  if (BIAS == kBiasRows) {
    const int rows_p = 2 * a.gh - 1 + 2 * kBiasPadRows;
    c.brs = make_rsrc(a.bias4 + static_cast<int64_t>(c.head) * rows_p * 4 * a.Lpad,
                      static_cast<uint32_t>(rows_p * 16 * a.Lpad));
    c.win_bytes = a.win_rows * 16 * a.Lpad;  // <= 8 KiB: two pieces per wave
  }
  c.drs = c.ars;
  c.dvoff = c.dld2 = 0;
  if (BIAS == kBiasDense) {
    // The range ends at the last real entry of this (b, h), so rows and
    // keys past N read 0 (rows past N are never stored, keys past N are
    // masked); every offset the copies form stays below 2^32.
    const int64_t b = c.bh / a.H;
    c.drs = make_rsrc(a.dense + b * a.dsb + static_cast<int64_t>(c.head) * a.dsh,
                      static_cast<uint32_t>(((a.N - 1) * a.dld + a.N) * 2));
    c.dld2 = static_cast<uint32_t>(a.dld * 2);
    const int l = c.lane;
    c.dvoff = static_cast<uint32_t>(c.q0 + (l >> 3)) * c.dld2 + static_cast<uint32_t>(((l & 7) ^ ((l >> 4) & 3)) * 16);
    // row r = 32 wave + li, group b of block 0 sits in chunk b ^ ((r/2) & 3)
    const int r = c.wave * 32 + c.li, x = (c.li >> 1) & 3;
#pragma unroll
    for (int b2 = 0; b2 < 4; ++b2) c.off_dn[b2] = r * 128 + ((b2 ^ x) << 4) + 8 * c.lh;
  }

  // ---- logit bound M (log2 units) ------------------------------------------
  const int nblk = a.Npad / 64;
  float km = 0.0f, bm = 0.0f;
  if (SMALL)
    km = kmax_small;
  else
    for (int e = c.tid; e < nblk; e += kThreads) km = fmaxf(km, a.kmax_blk[static_cast<int64_t>(c.bh) * nblk + e]);
  if (BIAS == kBiasRows) {
    const int rows = 2 * a.gh - 1;
    for (int e = c.tid; e < rows; e += kThreads) bm = fmaxf(bm, a.bias_row_max[c.head * rows + e]);
  } else if (BIAS == kBiasTable) {
    // the whole table goes to LDS once, as float32 * log2e
    const int n = (2 * a.gh - 1) * (2 * a.gw - 1);
    const uint16_t* t = a.table + static_cast<int64_t>(c.head) * n;
#pragma unroll 4
    for (int e = c.tid; e < n; e += kThreads) {
      const float v = kLog2e * bf16_to_f32(t[a.table_flip ? n - 1 - e : e]);  // flip: both axes
      c.table[e] = v;
      bm = fmaxf(bm, fabsf(v));
    }
    const int yc = c.yq < a.gh ? c.yq : a.gh - 1;
    c.fidx = (yc + a.gh - 1) * (2 * a.gw - 1) + c.xq + a.gw - 1;
  }
  const v3f mx = block_max3(km, bm, alpha_q, red);
  return a.qscale * mx[2] * mx[0] * static_cast<float>(a.d) + mx[1];
}

// A wave's 32 bf16 output rows staged in LDS (see fwd_epilogue): rows of
// C = d / 8 16-byte chunks, chunk j of row r at position j ^ (r & sw).
// out_stage_put stores channels c0..c0+3 of row li; out_stage_flush writes
// rows r0 .. r0+31 below N as whole chunks, nontemporal.
__device__ __forceinline__ void out_stage_put(unsigned char* ws, int li, int C, int sw, int c0, v2u w) {
  *reinterpret_cast<v2u*>(ws + (li * C + ((c0 >> 3) ^ (li & sw))) * 16 + (c0 & 4) * 2) = w;
}

__device__ __forceinline__ void out_stage_flush(const FwdArgs& a, const unsigned char* ws, int C, int sw, int lane,
                                                int64_t bidx, int head, int r0) {
  for (int e = lane; e < 32 * C; e += 64) {
    const int r = e / C, j = e - r * C;
    if (r0 + r < a.N) {
      const v4u x = lds_load<v4u>(ws, (r * C + (j ^ (r & sw))) * 16);
      __builtin_nontemporal_store(x, reinterpret_cast<v4u*>(a.o + token_offset(a.os, bidx, head, r0 + r) + 8 * j));
    }
  }
}

// O = O^T / l, bf16, one query per lane; the rows' log-sum-exp when asked.
// Without `stage` each lane stores its 4-channel pieces straight to HBM
// (8 bytes in each of 32 rows per instruction).  With `stage` (every wave of
// the workgroup calls it, at the end of its key loop) the wave's 32 rows go
// through LDS first: waves 0, 1 use stage0, waves 2, 3 stage1, 32 * d bf16
// each, rows of d / 8 16-byte chunks, chunk j of row r at position
// j ^ (r & 7) when d % 64 == 0 (conflict-free 8-byte writes and 16-byte
// reads).  The rows then leave as
// whole 16-byte chunks, 8 rows per instruction, in nontemporal stores that
// stream out while other workgroups still run.
template <int NCH, int CB, bool XONES>
__device__ __forceinline__ void fwd_epilogue(const Ctx<NCH>& c, const FwdArgs& a, Acc<CB, XONES>& acc, float mrow,
                                             unsigned char* stage0 = nullptr, unsigned char* stage1 = nullptr) {
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) pin_uniform(acc.o[cb]);
  float lsum;
  if (XONES) {
    lsum = acc.rs[0];
  } else {
    // rows d and d+4 of the last block: register 4 * ((d % 32) / 8)
    const int b1 = (a.d & 31) >> 3;
    const v16f& last = acc.o[CB - 1];
    lsum = b1 == 1 ? last[4] : (b1 == 2 ? last[8] : last[12]);
  }
  const float inv = 1.0f / lsum;
  // log2 of the softmax denominator, kept for the backward pass (0 for the
  // padding rows, which the backward reads as masked columns)
  if (a.lse && c.lh == 0) a.lse[c.tokbase + c.qi] = c.qi < a.N ? mrow + log2f(lsum) : 0.0f;
  if (a.lse_out && c.lh == 0 && c.qi < a.N)
    a.lse_out[static_cast<int64_t>(c.bh) * a.N + c.qi] = (mrow + log2f(lsum)) * kLn2;
  if (stage0 == nullptr) {
    if (c.qi < a.N) {
      uint16_t* orow = a.o + token_offset(a.os, c.bh / a.H, c.head, c.qi);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int c0 = cb * 32 + 8 * b + 4 * c.lh;
          if (c0 < a.d) {
            uint2 w;
            w.x = pack_bf16x2(acc.o[cb][4 * b + 0] * inv, acc.o[cb][4 * b + 1] * inv);
            w.y = pack_bf16x2(acc.o[cb][4 * b + 2] * inv, acc.o[cb][4 * b + 3] * inv);
            *reinterpret_cast<uint2*>(orow + c0) = w;
          }
        }
    }
    return;
  }
  // lane and wave recomputed here rather than kept live through the key loop
  const int lane = static_cast<int>(threadIdx.x & 63), li = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int C = a.d >> 3, sw = (C & 7) == 0 ? 7 : 0;
  unsigned char* ws = (wave < 2 ? stage0 : stage1) + (wave & 1) * 64 * a.d;
  __syncthreads();  // every wave is past its last read of the tile buffers
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c0 = cb * 32 + 8 * b + 4 * (lane >> 5);
      if (c0 < a.d) {
        v2u w;
        w[0] = pack_bf16x2(acc.o[cb][4 * b + 0] * inv, acc.o[cb][4 * b + 1] * inv);
        w[1] = pack_bf16x2(acc.o[cb][4 * b + 2] * inv, acc.o[cb][4 * b + 3] * inv);
        out_stage_put(ws, li, C, sw, c0, w);
      }
    }
  __syncthreads();
  out_stage_flush(a, ws, C, sw, lane, c.bh / a.H, c.head, c.q0 + wave * 32);
}

// Waves per SIMD the register budget is sized for (accumulator blocks, QK
// chunks).
template <int NB, int NCH = 1>
struct Occupancy {
  static constexpr int kWaves = fwd_waves_for_blocks(NB, NCH);
};

template <int NCH, int CB, bool XONES, int BIAS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Occupancy<CB + XONES, NCH>::kWaves)))
attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) TileBuf<NCH, CB, BIAS> tb0;
  __shared__ __attribute__((aligned(16))) TileBuf<NCH, CB, BIAS> tb1;
  __shared__ float red[kRedFloats];
  extern __shared__ __attribute__((aligned(16))) float s_table[];

  Ctx<NCH> c;
  const float M = workgroup_setup<NCH, CB, BIAS>(c, a, red, s_table);

  Acc<CB, XONES> acc;
  float mrow = 0.0f;  // the offset the row sums are taken against (log2 units)
  if constexpr (BIAS == kBiasDense) {
    // no bound on a dense bias short of reading all of it: exact softmax
    (void)M;
    mrow = run_exact_pass<NCH, CB, XONES, BIAS>(c, tb0, tb1, acc);
  } else {
    if (M <= kFastMaxLogit)  // false for NaN as well
      run_fast_pass<NCH, CB, XONES, BIAS>(c, tb0, tb1, acc);
    else
      mrow = run_exact_pass<NCH, CB, XONES, BIAS>(c, tb0, tb1, acc);
  }

  if constexpr (BIAS == kBiasDense || (CB != 1 && CB != 2 && CB != 4)) {
    // direct stores: staging costs these variants registers (spills) inside
    // the key loop
    fwd_epilogue<NCH, CB, XONES>(c, a, acc, mrow);
  } else {
    // waves 0, 1 stage their rows in tb0's V^T tile, waves 2, 3 in tb1's
    static_assert(sizeof(tb0.vt) >= 2 * 32 * (32 * CB) * 2, "two waves' output rows fit one V^T tile");
    fwd_epilogue<NCH, CB, XONES>(c, a, acc, mrow, reinterpret_cast<unsigned char*>(tb0.vt),
                                 reinterpret_cast<unsigned char*>(tb1.vt));
  }
}

// -------------------------------------------------- one launch, short N ---
// For N <= kSmallKeys and d in {32, 64} (table or no bias) a workgroup packs
// all keys and values of its head straight into LDS, in exactly the tile
// layouts the prologue writes and the copies bring (so the result is bit for
// bit the two-launch path's), and runs the key loop without copies: one
// launch instead of two and no round trip of the key operands and V^T
// through HBM.  Each head's K and V are read by its ceil(N / 128)
// workgroups.
constexpr int kSmallTiles = 4;
constexpr int kSmallKeys = kSmallTiles * kBN;

// Key (within its 64-key tile) that P.V slot `slot` of the V^T tile holds:
// slots 8h..8h+3 of a 16-slot group hold keys 4h..4h+3, slots 8h+4..8h+7
// keys 8+4h..8+4h+3 (the order in which a lane holds its keys after QK).
__device__ __forceinline__ int vt_slot_key_fwd(int slot) {
  const int g = slot >> 4, s16 = slot & 15, hh = s16 >> 3, s = s16 & 7;
  return g * 16 + (s < 4 ? 4 * hh + s : 8 + 4 * hh + (s - 4));
}

template <int CB, int BIAS>
__device__ __forceinline__ float pack_head(const FwdArgs& a, int bh, TileBuf<1, CB, BIAS>* tiles, float* red) {
  const int64_t b = bh / a.H, h = bh - b * a.H;
  const int nkt = (a.N + kBN - 1) / kBN;
  const int W = a.d / 32;
  float km = 0.0f;
  // keys: one task per (key, 32-channel word); the word's fp4 operand dwords
  // and its sum of |k| (chunk by chunk, in the prologue's order), the two
  // words of a key in lanes e and e ^ 1
  for (int e = threadIdx.x; e < nkt * kBN * 2; e += kThreads) {
    const int key = e >> 1, half = e & 1;
    uint32_t w = 0;
    float part = 0.0f;
    if (key < a.N && half < W) {
      const uint16_t* row = a.k + token_offset(a.ks, b, h, key) + 32 * half;
      float p[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) w |= chunk_signs(*reinterpret_cast<const uint4*>(row + 8 * kk), p[kk]) << (8 * kk);
      part = (p[0] + p[1]) + (p[2] + p[3]);
    }
    TileBuf<1, CB, BIAS>& tb = tiles[key >> 6];
    tb.k[(key & 63) * 2 + half] = expand_signs_fp4(w, fp4_magnitude(word_valid(a.d, half)));
    const float other = __shfl_xor(part, 1, 64);
    if (half == 0) {
      const float alpha = key < a.N ? (part + other) / static_cast<float>(a.d) : 0.0f;
      tb.ak[key & 63] = alpha;
      km = fmaxf(km, alpha);
      if (BIAS == kBiasTable) {
        const int j = key < a.N ? key : a.N - 1;
        const int yj = j / a.gw;
        tb.gk[key & 63] = yj * (2 * a.gw - 1) + (j - yj * a.gw);
      }
    }
  }
  // values: one task per (tile, 8-slot chunk q, 8-channel group g): the 8
  // keys of slots 8q..8q+7 are loaded, transposed in registers, and leave as
  // the 16-byte chunks q of rows 8g..8g+7 of V^T, chunk q of row c at
  // position q ^ ((c >> 1) & 7); padded keys give zeros
  const int C = a.d / 8;
  for (int e = threadIdx.x; e < nkt * 8 * C; e += kThreads) {
    const int t = e / (8 * C), r = e - t * 8 * C, q = r / C, g = r - q * C;
    uint4 x[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int key = t * kBN + vt_slot_key_fwd(8 * q + sl);
      x[sl] = key < a.N ? *reinterpret_cast<const uint4*>(a.v + token_offset(a.vs, b, h, key) + 8 * g)
                        : make_uint4(0u, 0u, 0u, 0u);
    }
    uint16_t* vt = tiles[t].vt;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 8 * g + i;
      // halfword i of each key's chunk; dword m = slots 2m, 2m + 1
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = (&x[2 * m].x)[i >> 1], hi = (&x[2 * m + 1].x)[i >> 1];
        w[m] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      *reinterpret_cast<uint4*>(vt + cc * kBN + ((q ^ ((cc >> 1) & 7)) << 3)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  return block_max(km, red);  // its barriers also publish the tiles
}

// One tile of the short-N loop (no copies, no barrier).
template <bool FIRST, bool FAST, int CB, int BIAS>
__device__ __forceinline__ void small_tile(const Ctx<1>& c, const TileBuf<1, CB, BIAS>& tb, int t,
                                           Acc<CB, true>& acc, PendingPV<CB>& pp, float& mrow) {
  const FwdArgs& a = *c.a;
  KeyPos kp;
  kp.k0 = t * kBN;
  kp.ky[0] = kp.ky[1] = kp.kx[0] = 0;
  kp.kx[1] = 32;
  if (kp.k0 + kBN <= a.N) {
    if (FAST) {
      pipelined_block<false, !FIRST, 1, CB, true, BIAS>(c, tb, kp, 0, pp, acc);
      pipelined_block<false, true, 1, CB, true, BIAS>(c, tb, kp, 1, pp, acc);
    } else {
      exact_block<false, !FIRST, 1, CB, true, BIAS>(c, tb, kp, 0, pp, acc, mrow);
      exact_block<false, true, 1, CB, true, BIAS>(c, tb, kp, 1, pp, acc, mrow);
    }
  } else {
    if (FAST) {
      pipelined_block<true, !FIRST, 1, CB, true, BIAS>(c, tb, kp, 0, pp, acc);
      pipelined_block<true, true, 1, CB, true, BIAS>(c, tb, kp, 1, pp, acc);
    } else {
      exact_block<true, !FIRST, 1, CB, true, BIAS>(c, tb, kp, 0, pp, acc, mrow);
      exact_block<true, true, 1, CB, true, BIAS>(c, tb, kp, 1, pp, acc, mrow);
    }
  }
}

template <bool FAST, int CB, int BIAS>
__device__ __forceinline__ float small_pass(const Ctx<1>& c, const TileBuf<1, CB, BIAS>* tiles, Acc<CB, true>& acc) {
  const FwdArgs& a = *c.a;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc.o[cb] = v16f{};
  acc.rs[0] = acc.rs[1] = 0.0f;
  float mrow = FAST ? 0.0f : -INFINITY;
  const int nkt = (a.N + kBN - 1) / kBN;
  PendingPV<CB> pp;
  small_tile<true, FAST, CB, BIAS>(c, tiles[0], 0, acc, pp, mrow);
  for (int t = 1; t < nkt; ++t) small_tile<false, FAST, CB, BIAS>(c, tiles[t], t, acc, pp, mrow);
#pragma unroll
  for (int i = 0; i < 2 * CB; ++i) pv_mfma<CB, true>(i, pp, acc);
  acc.rs[0] = sum_halves(acc.rs[0] + acc.rs[1]);
  return mrow;
}

template <int CB, int BIAS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Occupancy<CB + 1>::kWaves)))
attn_fwd_small_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) TileBuf<1, CB, BIAS> tiles[kSmallTiles];
  __shared__ float red[kRedFloats];
  extern __shared__ __attribute__((aligned(16))) float s_table[];
  int wg = blockIdx.x;
  if (a.xcd_remap) {
    const int per = a.nwg >> 3;
    wg = (wg & 7) * per + (wg >> 3);
  }
  const float kmax = pack_head<CB, BIAS>(a, wg / a.nqt, tiles, red);
  Ctx<1> c;
  const float M = workgroup_setup<1, CB, BIAS, true>(c, a, red, s_table, kmax);
  Acc<CB, true> acc;
  float mrow = 0.0f;
  if (M <= kFastMaxLogit)
    small_pass<true, CB, BIAS>(c, tiles, acc);
  else
    mrow = small_pass<false, CB, BIAS>(c, tiles, acc);
  // the output rows leave through LDS (tiles 0 and 1's V^T, free by then)
  fwd_epilogue<1, CB, true>(c, a, acc, mrow, reinterpret_cast<unsigned char*>(tiles[0].vt),
                            reinterpret_cast<unsigned char*>(tiles[1].vt));
}

int small_static_lds(int cb, int mode) {
  if (mode == kBiasTable)
    return cb == 1 ? static_cast<int>(sizeof(TileBuf<1, 1, kBiasTable>)) * kSmallTiles + kRedFloats * 4
                   : static_cast<int>(sizeof(TileBuf<1, 2, kBiasTable>)) * kSmallTiles + kRedFloats * 4;
  return cb == 1 ? static_cast<int>(sizeof(TileBuf<1, 1, kBiasNone>)) * kSmallTiles + kRedFloats * 4
                 : static_cast<int>(sizeof(TileBuf<1, 2, kBiasNone>)) * kSmallTiles + kRedFloats * 4;
}

bool small_supported(int64_t N, int d, int mode) {
  return N <= kSmallKeys && (d == 32 || d == 64) && (mode == kBiasNone || mode == kBiasTable);
}

int launch_attention_small(const FwdArgs& a, int mode, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.nwg), block(kThreads);
  const int lds = a.dyn_lds;
  const int cb = a.dpad / 32;
  if (cb == 1 && mode == kBiasTable) hipLaunchKernelGGL((attn_fwd_small_kernel<1, kBiasTable>), grid, block, lds, s, a);
  else if (cb == 1 && mode == kBiasNone) hipLaunchKernelGGL((attn_fwd_small_kernel<1, kBiasNone>), grid, block, lds, s, a);
  else if (cb == 2 && mode == kBiasTable) hipLaunchKernelGGL((attn_fwd_small_kernel<2, kBiasTable>), grid, block, lds, s, a);
  else if (cb == 2 && mode == kBiasNone) hipLaunchKernelGGL((attn_fwd_small_kernel<2, kBiasNone>), grid, block, lds, s, a);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

// ------------------------------------------------------ 8-bit P.V path ---
// The pages' hybrid quantization ("Cuantizacion Hibrida"): 1-bit Q and K,
// 8-bit attention coefficients and values.  Coefficients in [0, 1] take a
// static unsigned 8-bit code, values a per-channel signed 8-bit code:
//   code_ij = round-half-even(255 * 2^(s_ij - m_i)),  m_i = max_j s_ij,
//   O_ic    = s_c * sum_j code_ij vq_jc / sum_j code_ij.
// The codes are taken against the true row maximum, so a first pass over
// the keys finds m_i (QK and logits only), and the second forms the codes
// and runs P.V on v_mfma_i32_32x32x32_i8.  That instruction multiplies
// signed bytes, so the coefficient codes enter as code - 128 (the sign bit
// flipped) and the epilogue adds back 128 * sum_j vq_jc, a column sum of
// the value codes the prologue wrote: the integer product is exact.
constexpr float kLog2_255 = 7.994353436858858f;

template <int CB>
struct Acc8 {
  v16i o[CB];
};

__device__ __forceinline__ void pin_uniform_i(v16i& x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    int e = x[i];
    asm volatile("" : "+v"(e));
    x[i] = e;
  }
}

// One 64-key tile of the 8-bit path.  MAIN = false: running maximum of the
// logits only.  MAIN: the lane's 16 codes of each 32-key block, 4 per dword
// in the order the lane holds the keys (slot 16 lh + 4 g + i = key
// 8 g + 4 lh + i, the order of the value-code tile), the row sum of the
// codes, and the product with the value codes.
template <bool MAIN, bool MASK, int NCH, int CB, int BIAS>
__device__ __forceinline__ void int8_tile(const Ctx<NCH>& c, const TileBuf<NCH, CB, BIAS>& tb, const KeyPos& kp,
                                          float& mrow, float off, Acc8<CB>& acc, uint32_t& rsum, int nblk) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk >= nblk) break;  // uniform: the padded block of a ragged table-row tile
    v16f s = v16f{};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      s = mfma_signs_32x32x64(lds_load<v4i>(tb.k, c.off_k + ch * 2048 + blk * 1024), c.qop[ch], s);
    float sc[16];
    block_logits<MASK, NCH, CB, BIAS>(c, tb, kp, blk, s, sc);
    if (!MAIN) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mrow = fmaxf(mrow, sc[r]);
      continue;
    }
    v4i pb;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w = 0u;
      w = __builtin_amdgcn_cvt_pk_u8_f32(fast_exp2(sc[4 * g + 0] + off), 0, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(fast_exp2(sc[4 * g + 1] + off), 1, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(fast_exp2(sc[4 * g + 2] + off), 2, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(fast_exp2(sc[4 * g + 3] + off), 3, w);
      rsum = __builtin_amdgcn_udot4(w, 0x01010101u, rsum, false);
      pb[g] = static_cast<int>(w ^ 0x80808080u);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      acc.o[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(lds_load<v4i>(tb.vt, c.off8[blk] + cb * 2048), pb, acc.o[cb],
                                                         0, 0, 0);
  }
}

template <bool MAIN, int NCH, int CB, int BIAS>
__device__ __forceinline__ void int8_step(const Ctx<NCH>& c, const TileBuf<NCH, CB, BIAS>& cur,
                                          TileBuf<NCH, CB, BIAS>& nxt, int t, int nkt, KeyPos& kp, float& mrow,
                                          float off, Acc8<CB>& acc, uint32_t& rsum) {
  const FwdArgs& a = *c.a;
  const KeyPos kn = next_keys(kp, a.gw);
  if (t + 1 < nkt) copy_tile_async<NCH, CB, BIAS, MAIN ? kVInt8 : kVNone>(c, nxt, t + 1, kn);
  if (BIAS == kBiasRows)  // as in pass_step
    int8_tile<MAIN, false, NCH, CB, BIAS>(c, cur, kp, mrow, off, acc, rsum, kp.k0 + 32 < a.N ? 2 : 1);
  else if (kp.k0 + kBN <= a.N)
    int8_tile<MAIN, false, NCH, CB, BIAS>(c, cur, kp, mrow, off, acc, rsum, 2);
  else
    int8_tile<MAIN, true, NCH, CB, BIAS>(c, cur, kp, mrow, off, acc, rsum, 2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  kp = kn;
}

template <bool MAIN, int NCH, int CB, int BIAS>
__device__ __forceinline__ void int8_pass(const Ctx<NCH>& c, TileBuf<NCH, CB, BIAS>& tb0, TileBuf<NCH, CB, BIAS>& tb1,
                                          float& mrow, float off, Acc8<CB>& acc, uint32_t& rsum) {
  const FwdArgs& a = *c.a;
  KeyPos kp;
  kp.k0 = 0;
  kp.ky[0] = 0;
  kp.kx[0] = 0;
  kp.ky[1] = (BIAS == kBiasRows && a.gw == 32) ? 1 : 0;
  kp.kx[1] = (BIAS == kBiasRows && a.gw == 32) ? 0 : 32;
  copy_tile_async<NCH, CB, BIAS, MAIN ? kVInt8 : kVNone>(c, tb0, 0, kp);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nkt = (a.N + kBN - 1) / kBN;
  for (int t = 0; t < nkt; t += 2) {
    int8_step<MAIN, NCH, CB, BIAS>(c, tb0, tb1, t, nkt, kp, mrow, off, acc, rsum);
    if (t + 1 < nkt) int8_step<MAIN, NCH, CB, BIAS>(c, tb1, tb0, t + 1, nkt, kp, mrow, off, acc, rsum);
  }
}

template <int NCH, int CB, int BIAS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Occupancy<CB>::kWaves)))
attn_fwd_int8_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) TileBuf<NCH, CB, BIAS> tb0;
  __shared__ __attribute__((aligned(16))) TileBuf<NCH, CB, BIAS> tb1;
  __shared__ float red[kRedFloats];
  extern __shared__ __attribute__((aligned(16))) float s_table[];

  Ctx<NCH> c;
  (void)workgroup_setup<NCH, CB, BIAS>(c, a, red, s_table);
  // the value-code tiles of this (b, h): dpad rows of 64 bytes per tile
  constexpr int kV8Bytes = 32 * CB * kBN;
  c.vrs = make_rsrc(reinterpret_cast<const char*>(a.vq) + static_cast<int64_t>(c.bh) * (a.Npad / kBN) * kV8Bytes,
                    static_cast<uint32_t>((a.Npad / kBN) * kV8Bytes));
  {
    // operand of block b: row li (+ 32 cb), chunk (2 b + lh) ^ ((li / 4) & 3)
    const int x = (c.li >> 2) & 3;
#pragma unroll
    for (int b = 0; b < 2; ++b) c.off8[b] = c.li * 64 + (((2 * b + c.lh) ^ x) << 4);
  }

  Acc8<CB> acc;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc.o[cb] = v16i{};
  uint32_t rsum = 0u;
  float mrow = -INFINITY;
  int8_pass<false, NCH, CB, BIAS>(c, tb0, tb1, mrow, 0.0f, acc, rsum);
  mrow = max_halves(mrow);
  // exp2(s + off) = 255 * 2^(s - m): the row maximum gets code 255
  int8_pass<true, NCH, CB, BIAS>(c, tb0, tb1, mrow, kLog2_255 - mrow, acc, rsum);

  // ---- epilogue: O = s_c (acc + 128 colsum_c) / sum of codes, bf16 --------
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) pin_uniform_i(acc.o[cb]);
  const auto pr = __builtin_amdgcn_permlane32_swap(rsum, rsum, false, false);
  const float inv = 1.0f / static_cast<float>(pr[0] + pr[1]);
  const float* vsc = a.vscale + static_cast<int64_t>(c.bh) * a.dpad;
  const int* vcs = a.vcsum + static_cast<int64_t>(c.bh) * a.dpad;
  // channels c0..c0+3 of the lane's row, packed to bf16
  auto out4 = [&](int cb, int b, int c0) {
    const v4f sv = *reinterpret_cast<const v4f*>(vsc + c0);
    const v4i cs = *reinterpret_cast<const v4i*>(vcs + c0);
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<float>(acc.o[cb][4 * b + i] + 128 * cs[i]) * sv[i] * inv;
    return v2u{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  };
  if constexpr (CB == 1 || CB == 2 || CB == 4) {
    // the rows leave through LDS as in fwd_epilogue: waves 0, 1 in tb0's
    // V^T tile, waves 2, 3 in tb1's (rows past N are formed but not written)
    static_assert(sizeof(tb0.vt) >= 2 * 32 * (32 * CB) * 2, "two waves' output rows fit one V^T tile");
    const int lane = static_cast<int>(threadIdx.x & 63), li = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int C = a.d >> 3, sw = (C & 7) == 0 ? 7 : 0;
    unsigned char* ws = reinterpret_cast<unsigned char*>(wave < 2 ? tb0.vt : tb1.vt) + (wave & 1) * 64 * a.d;
    __syncthreads();  // every wave is past its last read of the tile buffers
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c0 = cb * 32 + 8 * b + 4 * (lane >> 5);
        if (c0 < a.d) out_stage_put(ws, li, C, sw, c0, out4(cb, b, c0));
      }
    __syncthreads();
    out_stage_flush(a, ws, C, sw, lane, c.bh / a.H, c.head, c.q0 + wave * 32);
  } else if (c.qi < a.N) {
    uint16_t* orow = a.o + token_offset(a.os, c.bh / a.H, c.head, c.qi);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c0 = cb * 32 + 8 * b + 4 * c.lh;
        if (c0 < a.d) *reinterpret_cast<v2u*>(orow + c0) = out4(cb, b, c0);
      }
  }
}

// ================================================================ backward ==
// Gradients of the forward for an output gradient dO, with the reading of
// the sign gradient (alpha = mean |x| differentiated exactly, sign through
// the clipped straight-through estimator).  With P = softmax(S), rebuilt
// from the forward's log2-sum-exp2, and delta_i = <dO_i, O_i>:
//   dP_ij = <dO_i, V_j>,   dS_ij = P_ij (dP_ij - delta_i),
//   dq~_i = scale sum_j dS_ij alpha_k,j sign(k_j),
//   dk~_j = scale sum_i dS_ij alpha_q,i sign(q_i),   dV_j = sum_i P_ij dO_i,
//   dx = sign(x) <sign(x), dx~> / d + alpha_x 1{|x| <= 1} dx~  (x = q, k).
// One kernel, two roles.  kRoleQ: a lane holds a query, the columns are the
// keys (the forward's layout).  kRoleKV: a lane holds a key, the columns are
// the queries; with queries and keys exchanged the bias is the same
// relative-position form with the table flipped in both axes, so the
// forward's setup, tile copies and logits serve both.  Per 32-column block:
// S on the fp4 unit as in the forward; dP (rows = columns, one row token
// per lane, like S) on bf16 MFMA from a natural [64][d] tile of V or dO and
// the lane's own dO or V row; then the products that sum over the columns,
// on bf16 MFMA with the column tiles transposed as the forward's V^T: the
// +/-1 signs of K (kRoleQ), dO^T and the +/-1 signs of Q (kRoleKV).
template <int ROLE, int NCH, int CB, int BIAS>
struct BwdTileBuf {
  v4i k[NCH * kBN * 2];                         // column fp4 operands
  float ak[kBN];                                 // column scales
  int gk[BiasSizes<BIAS>::kGk];                  // grid offsets (table mode)
  float cl[kBN];                                 // kRoleKV: columns' log2-sum-exp2
  float cd[kBN];                                 // kRoleKV: columns' delta
  uint16_t y[kBN * 32 * CB];                     // natural tile [64][dpad]
  uint16_t vt[32 * CB * kBN];                    // K signs (kRoleQ) / dO^T (kRoleKV)
  uint16_t vt2[ROLE == kRoleKV ? 32 * CB * kBN : 8];  // Q signs (kRoleKV)
  float win[BiasSizes<BIAS>::kWin];              // bias window (table-row mode)
  // kRoleQ, table rows: this tile's table-gradient window, win_rows rows of
  // 2gw-1 entries (row = (yq - yq_lo) + (yk_hi - yk), column = xq - xk + gw - 1)
  float dwin[ROLE == kRoleQ && BIAS == kBiasRows ? kMaxWindowFloats : 4];
};

// Buffer resources of the backward's own column copies.
struct BwdCtx {
  rsrc_t zrs, z2rs, yrs, lrs, drs;
  int dtk;  // table mode: the table gradient is summed in LDS as round(dS 2^dtk)
};

// 16-byte chunk position of chunk `ch` of row `row` in the natural tile
// (C = 4 CB chunks per row): the XOR spreads the 16 rows that one
// quarter-wave reads over 16 different bank groups.
template <int CB>
__device__ __forceinline__ int ychunk(int row, int ch) {
  constexpr int C = 4 * CB;
  constexpr int sh = CB == 1 ? 2 : (CB == 2 ? 1 : 0);
  return ch ^ ((row >> sh) & (C - 1));
}

template <int ROLE, int NCH, int CB, int BIAS>
__device__ __forceinline__ void bwd_copy(const Ctx<NCH>& c, const BwdCtx& bc, BwdTileBuf<ROLE, NCH, CB, BIAS>& tb,
                                         int t, const KeyPos& kp) {
  copy_tile_async<NCH, CB, BIAS, kVNone>(c, tb, t, kp);
  constexpr int kTBytes = 32 * CB * kBN * 2;
  const uint32_t loff = static_cast<uint32_t>(c.wave * 1024 + c.lane * 16);
#pragma unroll
  for (int j = 0; j < kTBytes / 4096; ++j) {
    dma16(bc.zrs, reinterpret_cast<char*>(&tb.vt[0]) + (c.wave + 4 * j) * 1024, loff,
          static_cast<uint32_t>(t * kTBytes + j * 4096));
    if (ROLE == kRoleKV)
      dma16(bc.z2rs, reinterpret_cast<char*>(&tb.vt2[0]) + (c.wave + 4 * j) * 1024, loff,
            static_cast<uint32_t>(t * kTBytes + j * 4096));
  }
  if (ROLE == kRoleKV) {
    if (c.wave == 1) dma4(bc.lrs, &tb.cl[0], static_cast<uint32_t>(c.lane * 4), static_cast<uint32_t>(kp.k0 * 4));
    if (c.wave == 2) dma4(bc.drs, &tb.cd[0], static_cast<uint32_t>(c.lane * 4), static_cast<uint32_t>(kp.k0 * 4));
  }
  // natural tile: rows k0 .. k0 + 63 of [N][d], 4 CB pieces of 1 KiB; every
  // offset is in the per-lane part, so rows past N fall outside the range
  // and read 0
  constexpr int C = 4 * CB, lgC = CB == 1 ? 2 : (CB == 2 ? 3 : 4);
  const int d = c.a->d;
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int m = c.wave + 4 * j;
    const int row = (64 * m + c.lane) >> lgC, pos = c.lane & (C - 1);
    const int ch = ychunk<CB>(row, pos);  // the XOR is its own inverse
    const uint32_t voff = static_cast<uint32_t>(((kp.k0 + row) * d + ch * 8) * 2);
    dma16(bc.yrs, reinterpret_cast<char*>(&tb.y[0]) + m * 1024, voff, 0u);
  }
}

template <int ROLE, int CB>
struct BwdAcc {
  v16f a1[CB];                         // dq~ (kRoleQ) or dk~ (kRoleKV), O^T-like layout
  v16f a2[ROLE == kRoleKV ? CB : 1];   // dv (kRoleKV)
};

// The last products of a finished block wait in registers (its bf16 dS * scale
// and P, and their operand tiles) and are issued after the next block's QK,
// so they run while that block's vector work goes on, as in the forward's
// pipeline: dq~ += (alpha dS) sign K (kRoleQ); dv += P^T dO and
// dk~ += (alpha dS^T) sign Q (kRoleKV).
template <int ROLE, int CB>
struct BwdPending {
  uint32_t ww[8];                                  // bf16 dS * the other side's scale
  uint32_t pw[ROLE == kRoleKV ? 8 : 1];            // bf16 P (kRoleKV)
  v8bf vop[2][CB];                                 // K signs (kRoleQ) / dO^T (kRoleKV)
  v8bf vop2[ROLE == kRoleKV ? 2 : 1][ROLE == kRoleKV ? CB : 1];  // Q signs (kRoleKV)
};

// Where the held operands fit the register budget: table rows, and the
// query role at d <= 64.  Elsewhere each block issues its products at its
// end (holding them spilled registers to scratch).
template <int ROLE, int NCH, int BIAS>
constexpr bool bwd_pipelined() { return BIAS == kBiasRows || (ROLE == kRoleQ && NCH == 1); }

template <int ROLE, int CB>
__device__ __forceinline__ void bwd_pending_mfma(const BwdPending<ROLE, CB>& pd, BwdAcc<ROLE, CB>& acc) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const v4u wv = {pd.ww[4 * half], pd.ww[4 * half + 1], pd.ww[4 * half + 2], pd.ww[4 * half + 3]};
    const v8bf wop = __builtin_bit_cast(v8bf, wv);
    if (ROLE == kRoleQ) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc.a1[cb] = mfma_bf16_32x32x16(pd.vop[half][cb], wop, acc.a1[cb]);
    } else {
      const v4u pv = {pd.pw[4 * half], pd.pw[4 * half + 1], pd.pw[4 * half + 2], pd.pw[4 * half + 3]};
      const v8bf pop = __builtin_bit_cast(v8bf, pv);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        acc.a2[cb] = mfma_bf16_32x32x16(pd.vop[half][cb], pop, acc.a2[cb]);
        acc.a1[cb] = mfma_bf16_32x32x16(pd.vop2[ROLE == kRoleKV ? half : 0][ROLE == kRoleKV ? cb : 0], wop,
                                        acc.a1[cb]);
      }
    }
  }
}

// Diagonal sums of one 32x32 block of dS in the MFMA result layout (lane
// l = 32 lh + li holds query li; register r = 4 g + i holds key
// j = 8 g + 4 lh + i).  Returns, in lane t, the sum of dS[li][j] over
// li - j = t - 32 (lane 0, diagonal -32, is always 0).
//
// Write li = 16 qh + L (qh: the lane's row of 16 within its half) and
// j = 16 kh + 8 (g & 1) + 4 lh + i.  Shifting register r left inside the
// 16-lane rows by s = 8 (g & 1) + i brings the keys of one diagonal into one
// lane: lane L then holds diagonal 16 (qh - kh) + L - 4 lh, and the values
// that leave the row (shifted the other way, by 16 - s) diagonal
// 16 (qh - kh - 1) + L - 4 lh.  So three accumulators a[e], e = kh or kh + 1,
// each hold diagonal 16 (qh - e) + L - 4 lh in lane L.  The upper half is
// then moved 4 lanes down (what leaves its rows goes to a[e + 1]; a[2]'s
// lanes 0..3 there are empty), after which a[e] in rows (lh, qh) belongs to
// output row qh - e + 2 in both halves, and two lane-half swaps and one row
// swap put every partial sum in its lane.
__device__ __forceinline__ float diagonal_sums(const float (&x)[16]) {
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f;
#define BA_DIAG_STEP(R, S, LO, HI)                 \
  LO += row_shl_c<S>(0.0f, x[R]);                  \
  HI += row_shr_c<16 - S>(0.0f, x[R]);
  a0 += x[0];
  BA_DIAG_STEP(1, 1, a0, a1)
  BA_DIAG_STEP(2, 2, a0, a1)
  BA_DIAG_STEP(3, 3, a0, a1)
  BA_DIAG_STEP(4, 8, a0, a1)
  BA_DIAG_STEP(5, 9, a0, a1)
  BA_DIAG_STEP(6, 10, a0, a1)
  BA_DIAG_STEP(7, 11, a0, a1)
  a1 += x[8];
  BA_DIAG_STEP(9, 1, a1, a2)
  BA_DIAG_STEP(10, 2, a1, a2)
  BA_DIAG_STEP(11, 3, a1, a2)
  BA_DIAG_STEP(12, 8, a1, a2)
  BA_DIAG_STEP(13, 9, a1, a2)
  BA_DIAG_STEP(14, 10, a1, a2)
  BA_DIAG_STEP(15, 11, a1, a2)
#undef BA_DIAG_STEP
  // upper half (rows 2, 3): 4 lanes down, the overflow into the next e
  a2 = row_shl_c<4, 0xC>(a2, a2) + row_shr_c<12, 0xC>(0.0f, a1);
  a1 = row_shl_c<4, 0xC>(a1, a1) + row_shr_c<12, 0xC>(0.0f, a0);
  a0 = row_shl_c<4, 0xC>(a0, a0);
  // e = 2 to output rows 0, 1 and e = 0 to rows 2, 3 (sums of both halves)
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a2), __float_as_uint(a0), false, false);
  const float u = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  // e = 1: rows (qh = 0) to output row 1, (qh = 1) to output row 2
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a1), __float_as_uint(a1), false, false);
  const auto r = __builtin_amdgcn_permlane32_swap(q[0], q[1], false, false);
  return u + rows_only<0x6>(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// The table gradient (kRoleQ, want_dt).  Table-row mode: a wave's 32 queries
// and a block's 32 keys each lie in one grid row, so the block adds its 63
// diagonal sums (diagonal_sums) to consecutive entries of one row of this
// wave's window; dsk/dbase keep the sums and the window position, and
// bwd_step adds them once the tile's copies have landed.  Table mode: every
// dS_ij is added at the entry of its grid offset in a copy of the whole
// table that follows the table in dynamic LDS, as the integer round(dS 2^dtk)
// with an integer LDS add (float LDS adds run several times slower); dtk
// keeps the workgroup's sums below 2^30 (see attn_bwd_kernel).
template <int ROLE, bool MASK, int NCH, int CB, int BIAS>
__device__ __forceinline__ void bwd_tile(const Ctx<NCH>& c, BwdTileBuf<ROLE, NCH, CB, BIAS>& tb,
                                         const KeyPos& kp, const v8bf (&xop)[2 * CB], float lrow, float drow,
                                         BwdAcc<ROLE, CB>& acc, int nblk, bool want_dt, float (&dsk)[2],
                                         int (&dbase)[2], int dtk, BwdPending<ROLE, CB>& pd, bool& pending) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk >= nblk) break;  // uniform: the padded block of a ragged table-row tile
    v16f s = v16f{};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
      s = mfma_signs_32x32x64(lds_load<v4i>(tb.k, c.off_k + ch * 2048 + blk * 1024), c.qop[ch], s);
    if (pending) bwd_pending_mfma<ROLE, CB>(pd, acc);  // uniform: false for the first block only
    float sc[16];
    block_logits<MASK, NCH, CB, BIAS>(c, tb, kp, blk, s, sc);
    // dP: rows = the block's columns, one row token per lane
    v16f dp = v16f{};
    const int yrow = blk * 32 + c.li;
#pragma unroll
    for (int t = 0; t < 2 * CB; ++t)
      dp = mfma_bf16_32x32x16(lds_load<v8bf>(tb.y, (yrow * 4 * CB + ychunk<CB>(yrow, 2 * t + c.lh)) * 16), xop[t], dp);
    const float akv = lds_load<float>(tb.ak, c.off_akb + blk * 128);
    float clv = 0.0f, cdv = 0.0f;
    if (ROLE == kRoleKV) {
      clv = lds_load<float>(tb.cl, c.off_akb + blk * 128);
      cdv = lds_load<float>(tb.cd, c.off_akb + blk * 128);
    }
    uint32_t pw[8], ww[8];
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0, p1, d0, d1;
      if (ROLE == kRoleQ) {
        p0 = fast_exp2(sc[r] - lrow);
        p1 = fast_exp2(sc[r + 1] - lrow);
        d0 = p0 * (dp[r] - drow);
        d1 = p1 * (dp[r + 1] - drow);
      } else {
        p0 = fast_exp2(sc[r] - row_bcast(clv, r));
        p1 = fast_exp2(sc[r + 1] - row_bcast(clv, r + 1));
        d0 = p0 * (dp[r] - row_bcast(cdv, r));
        d1 = p1 * (dp[r + 1] - row_bcast(cdv, r + 1));
      }
      ww[r / 2] = pack_bf16x2(d0 * row_bcast(akv, r), d1 * row_bcast(akv, r + 1));
      pw[r / 2] = pack_bf16x2(p0, p1);
      dsv[r] = d0;
      dsv[r + 1] = d1;
    }
    if (ROLE == kRoleQ && BIAS == kBiasRows && want_dt) {
      // window row ky[1] - ky[blk]; diagonal 0 (query column xq - li, key
      // column kx[blk]) at column xq - li - kx[blk] + gw - 1
      const FwdArgs& a = *c.a;
      dbase[blk] = (kp.ky[1] - kp.ky[blk]) * (2 * a.gw - 1) + (c.xq - c.li - kp.kx[blk] + a.gw - 1);
      dsk[blk] = diagonal_sums(dsv);
    }
    if (ROLE == kRoleQ && BIAS == kBiasTable && want_dt) {
      const FwdArgs& a = *c.a;
      int* tacc = reinterpret_cast<int*>(c.table + (2 * a.gh - 1) * (2 * a.gw - 1)) + c.fidx;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const v4i g = lds_load<v4i>(tb.gk, c.off_gk + (blk * 32 + 8 * b) * 4);
        atomicAdd(tacc - g.x, __float2int_rn(ldexpf(dsv[4 * b + 0], dtk)));
        atomicAdd(tacc - g.y, __float2int_rn(ldexpf(dsv[4 * b + 1], dtk)));
        atomicAdd(tacc - g.z, __float2int_rn(ldexpf(dsv[4 * b + 2], dtk)));
        atomicAdd(tacc - g.w, __float2int_rn(ldexpf(dsv[4 * b + 3], dtk)));
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // this block becomes pending: its operand tiles leave LDS now, so the
      // pipeline runs across tile barriers
      const int pidx = 2 * blk + half;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        pd.vop[half][cb] = lds_load<v8bf>(tb.vt, c.off_v[pidx] + cb * 4096);
        if (ROLE == kRoleKV)
          pd.vop2[ROLE == kRoleKV ? half : 0][ROLE == kRoleKV ? cb : 0] =
              lds_load<v8bf>(tb.vt2, c.off_v[pidx] + cb * 4096);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pd.ww[j] = ww[j];
      if (ROLE == kRoleKV) pd.pw[ROLE == kRoleKV ? j : 0] = pw[j];
    }
    if (!bwd_pipelined<ROLE, NCH, BIAS>()) bwd_pending_mfma<ROLE, CB>(pd, acc);
    pending = bwd_pipelined<ROLE, NCH, BIAS>();
  }
}

// Table-row mode: each wave owns kWaveWindow floats of the tile's window
// buffer, two rows of 2gw - 1 entries (the rows ky[1] and ky[1] - 1 of the
// tile's keys, against the wave's one query row).
constexpr int kWaveWindow = kMaxWindowFloats / 4;

// Adds a tile's four wave windows into this workgroup's share of the table
// gradient (no other workgroup touches it: plain loads and stores, ordered by
// the tile barriers) and clears them.  kp: that tile's key position.  Entry
// (row, col) of the workgroup's window, row = (yq - yq_lo) + (ky[1] - yk),
// sums row row - (yq - yq_lo) of every wave window that has it; it belongs
// to share row gh - 1 - ky[1] + row.
template <int NCH>
__device__ __forceinline__ void flush_dwin(const Ctx<NCH>& c, float* dwin, const KeyPos& kp, float* share, int prow) {
  const FwdArgs& a = *c.a;
  const int w2 = 2 * a.gw - 1;
  const int r0 = a.gh - 1 - kp.ky[1];  // share row of window row 0
  int wrow[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) wrow[w] = (c.q0 + 32 * w) / a.gw - c.yq_lo;
  for (int e = c.tid; e < a.win_rows * w2; e += kThreads) {
    const int rw = e / w2, col = e - rw * w2, r = r0 + rw;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int rr = rw - wrow[w];
      if (rr == 0 || rr == 1) {
        float* p = dwin + w * kWaveWindow + rr * w2 + col;
        v += *p;
        *p = 0.0f;
      }
    }
    if (v != 0.0f && r >= 0 && r < prow) share[r * w2 + col] += v;
  }
}

template <int ROLE, int NCH, int CB, int BIAS>
__device__ __forceinline__ void bwd_step(const Ctx<NCH>& c, const BwdCtx& bc, const BwdArgs& ba,
                                         BwdTileBuf<ROLE, NCH, CB, BIAS>& cur,
                                         BwdTileBuf<ROLE, NCH, CB, BIAS>& nxt, int t, int nkt, KeyPos& kp,
                                         KeyPos& kprev, const v8bf (&xop)[2 * CB], float lrow, float drow,
                                         BwdAcc<ROLE, CB>& acc, float* share, BwdPending<ROLE, CB>& pd,
                                         bool& pending) {
  const FwdArgs& a = *c.a;
  const KeyPos kn = next_keys(kp, a.gw);
  // the previous tile's window sits in nxt; it is added to the share before
  // the next copies into nxt start (no copy is in flight here)
  if (ROLE == kRoleQ && BIAS == kBiasRows && ba.dtable && t > 0) flush_dwin(c, nxt.dwin, kprev, share, ba.prow);
  if (t + 1 < nkt) bwd_copy<ROLE, NCH, CB, BIAS>(c, bc, nxt, t + 1, kn);
  const bool want_dt = ROLE == kRoleQ && ba.dtable != nullptr;
  float dsk[2] = {0.0f, 0.0f};
  int dbase[2] = {0, 0};
  const int nb = BIAS == kBiasRows ? (kp.k0 + 32 < a.N ? 2 : 1) : 2;
  if (BIAS == kBiasRows)  // as in pass_step
    bwd_tile<ROLE, false, NCH, CB, BIAS>(c, cur, kp, xop, lrow, drow, acc, nb, want_dt, dsk, dbase, bc.dtk, pd, pending);
  else if (kp.k0 + kBN <= a.N)
    bwd_tile<ROLE, false, NCH, CB, BIAS>(c, cur, kp, xop, lrow, drow, acc, 2, want_dt, dsk, dbase, bc.dtk, pd, pending);
  else
    bwd_tile<ROLE, true, NCH, CB, BIAS>(c, cur, kp, xop, lrow, drow, acc, 2, want_dt, dsk, dbase, bc.dtk, pd, pending);
  __builtin_amdgcn_s_waitcnt(0);
  if (ROLE == kRoleQ && BIAS == kBiasRows && want_dt && c.lane != 0) {
    // lane t: diagonal t - 32 (lane 0 holds the empty diagonal -32); the
    // wave's own window, so plain read-modify-writes in program order
    float* wwin = cur.dwin + c.wave * kWaveWindow + c.lane - 32;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (blk >= nb) break;
      wwin[dbase[blk]] += dsk[blk];
    }
  }
  __syncthreads();
  kprev = kp;
  kp = kn;
}

// dx = sign(x) <sign(x), dx~> / d + alpha 1{|x| <= 1} dx~ for the lane's row
// token x, whose dx~ / scale sits in acc, stored as float32.
template <int CB>
__device__ __forceinline__ void binarize_back_store(bool valid, const uint16_t* xr, float alpha, int d, int lh,
                                                    float scale, const v16f (&acc)[CB], float* out) {
  float dot = 0.0f;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c0 = cb * 32 + 8 * b + 4 * lh;
      const uint2 raw = valid ? *reinterpret_cast<const uint2*>(xr + c0) : make_uint2(0u, 0u);
      const uint32_t w2[2] = {raw.x, raw.y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = bf16_to_f32(static_cast<uint16_t>(e & 1 ? w2[e >> 1] >> 16 : w2[e >> 1] & 0xffffu));
        dot += (x < 0.0f ? -1.0f : 1.0f) * acc[cb][4 * b + e];
      }
    }
  dot = sum_halves(dot) * scale / static_cast<float>(d);
  if (!valid) return;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c0 = cb * 32 + 8 * b + 4 * lh;
      const uint2 raw = *reinterpret_cast<const uint2*>(xr + c0);
      const uint32_t w2[2] = {raw.x, raw.y};
      v4f o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = bf16_to_f32(static_cast<uint16_t>(e & 1 ? w2[e >> 1] >> 16 : w2[e >> 1] & 0xffffu));
        const float g = scale * acc[cb][4 * b + e];
        o[e] = (x < 0.0f ? -dot : dot) + (fabsf(x) <= 1.0f ? alpha * g : 0.0f);
      }
      *reinterpret_cast<v4f*>(out + c0) = o;
    }
}

// Waves per SIMD the backward's register budget is sized for.  At d = 128
// (two QK chunks) the tiles take 75-125 KB of LDS, one or two workgroups per
// CU; held to 256 registers the query-role variants spilled 55 and 71 of
// them, and at one wave they run 19-22 % faster.  The d <= 64 variants keep
// two waves (their few spills cost less than half the occupancy).
template <int NCH>
struct BwdOcc {
  static constexpr int kWaves = NCH == 2 ? 1 : 2;
};

template <int ROLE, int NCH, int CB, int BIAS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BwdOcc<NCH>::kWaves)))
attn_bwd_kernel(BwdArgs ba) {
  __shared__ __attribute__((aligned(16))) BwdTileBuf<ROLE, NCH, CB, BIAS> tb0;
  __shared__ __attribute__((aligned(16))) BwdTileBuf<ROLE, NCH, CB, BIAS> tb1;
  __shared__ float red[kRedFloats];
  extern __shared__ __attribute__((aligned(16))) float s_table[];
  const FwdArgs& a = ba.f;

  Ctx<NCH> c;
  (void)workgroup_setup<NCH, CB, BIAS>(c, a, red, s_table);
  const int64_t bhN = static_cast<int64_t>(c.bh) * a.N;
  BwdCtx bc;
  constexpr int kTBytes = 32 * CB * kBN * 2;
  const int ntile = a.Npad / kBN;
  bc.zrs = make_rsrc(reinterpret_cast<const char*>(ba.zt) + static_cast<int64_t>(c.bh) * ntile * kTBytes,
                     static_cast<uint32_t>(ntile * kTBytes));
  bc.z2rs = bc.zrs;
  if (ROLE == kRoleKV)
    bc.z2rs = make_rsrc(reinterpret_cast<const char*>(ba.zt2) + static_cast<int64_t>(c.bh) * ntile * kTBytes,
                        static_cast<uint32_t>(ntile * kTBytes));
  bc.yrs = make_rsrc(ba.ynat + bhN * a.d, static_cast<uint32_t>(a.N * a.d * 2));
  bc.lrs = make_rsrc(ba.lse + c.tokbase, static_cast<uint32_t>(a.Npad * 4));
  bc.drs = make_rsrc(ba.delta + c.tokbase, static_cast<uint32_t>(a.Npad * 4));

  // the lane's dP operand: its dO row (kRoleQ) or V row (kRoleKV), 8
  // channels per 16-channel step
  const bool valid = c.qi < a.N;
  const uint16_t* xr = ba.xrow + (bhN + (valid ? c.qi : 0)) * a.d;
  v8bf xop[2 * CB];
#pragma unroll
  for (int t = 0; t < 2 * CB; ++t) {
    const uint4 raw = valid ? *reinterpret_cast<const uint4*>(xr + 16 * t + 8 * c.lh) : make_uint4(0u, 0u, 0u, 0u);
    xop[t] = __builtin_bit_cast(v8bf, raw);
  }
  float lrow = 0.0f, drow = 0.0f;
  if (ROLE == kRoleQ) {
    // the row's log2-sum-exp2 and delta_i = <dO_i, O_i> (0 past N), both
    // written before this launch
    lrow = ba.lse[c.tokbase + c.qi];
    drow = ba.delta[c.tokbase + c.qi];
  }

  BwdAcc<ROLE, CB> acc;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    acc.a1[cb] = v16f{};
    if (ROLE == kRoleKV) acc.a2[cb] = v16f{};
  }
  KeyPos kp;
  kp.k0 = 0;
  kp.ky[0] = 0;
  kp.kx[0] = 0;
  kp.ky[1] = (BIAS == kBiasRows && a.gw == 32) ? 1 : 0;
  kp.kx[1] = (BIAS == kBiasRows && a.gw == 32) ? 0 : 32;
  // table-gradient accumulators start at zero; this workgroup's share of
  // the table gradient (table rows: cleared here, added to per tile)
  const int tsize = (2 * a.gh - 1) * (2 * a.gw - 1);
  float* share = nullptr;
  if (ROLE == kRoleQ && ba.dtable) {
    share = ba.dtpart + (static_cast<int64_t>(c.bh) * a.nqt + c.q0 / kBM) * ba.prow * (2 * a.gw - 1);
    if (BIAS == kBiasRows) {
      for (int e = c.tid; e < kMaxWindowFloats; e += kThreads) tb0.dwin[e] = tb1.dwin[e] = 0.0f;
      for (int e = c.tid; e < ba.prow * (2 * a.gw - 1); e += kThreads) share[e] = 0.0f;
    }
    if (BIAS == kBiasTable)
      for (int e = c.tid; e < tsize; e += kThreads) c.table[tsize + e] = 0.0f;
  }
  // Table mode: the scale of the integer sums.  With P <= 1, |dP_ij| and
  // |delta_i| both at most |dO_i|_1 max|v|, so |dS_ij| <= 2 |dO_i|_1 max|v|,
  // and a query meets each grid offset at most once: every entry's sum over
  // this workgroup is below B = 2 max|v| sum_i |dO_i|_1.  2^dtk B < 2^30, so
  // no sum overflows, and each rounds by at most 64 2^-dtk, below 1e-7 B.
  bc.dtk = 0;
  if (ROLE == kRoleQ && BIAS == kBiasTable && ba.dtable) {
    float l1 = 0.0f;
#pragma unroll
    for (int t = 0; t < 2 * CB; ++t) {
      const uint4 rg = __builtin_bit_cast(uint4, xop[t]);
      const uint32_t wg[4] = {rg.x, rg.y, rg.z, rg.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        l1 += fabsf(bf16_to_f32(static_cast<uint16_t>(wg[e] & 0xffffu))) + fabsf(bf16_to_f32(static_cast<uint16_t>(wg[e] >> 16)));
    }
    const float dsum = block_sum(l1, red);  // both halves of every query's row
    float vm = 0.0f;
    for (int t = c.tid; t < ntile; t += kThreads) vm = fmaxf(vm, ba.vmax[static_cast<int64_t>(c.bh) * ntile + t]);
    const float bound = 2.0f * block_max(vm, red) * dsum;
    if (bound > 0.0f && bound < INFINITY) bc.dtk = 29 - ilogbf(bound);
  }
  bwd_copy<ROLE, NCH, CB, BIAS>(c, bc, tb0, 0, kp);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nkt = (a.N + kBN - 1) / kBN;
  KeyPos kprev = kp;
  BwdPending<ROLE, CB> pd;
  bool pending = false;
  for (int t = 0; t < nkt; t += 2) {
    bwd_step<ROLE, NCH, CB, BIAS>(c, bc, ba, tb0, tb1, t, nkt, kp, kprev, xop, lrow, drow, acc, share, pd, pending);
    if (t + 1 < nkt)
      bwd_step<ROLE, NCH, CB, BIAS>(c, bc, ba, tb1, tb0, t + 1, nkt, kp, kprev, xop, lrow, drow, acc, share, pd,
                                    pending);
  }
  if (pending) bwd_pending_mfma<ROLE, CB>(pd, acc);  // the last block's products
  if (ROLE == kRoleQ && ba.dtable) {
    // the last tile's window (rows), or the whole table (table mode)
    if (BIAS == kBiasRows) flush_dwin(c, (nkt & 1) ? tb0.dwin : tb1.dwin, kprev, share, ba.prow);
    if (BIAS == kBiasTable) {
      const int* tsum = reinterpret_cast<const int*>(c.table + tsize);
      for (int e = c.tid; e < tsize; e += kThreads) share[e] = ldexpf(static_cast<float>(tsum[e]), -bc.dtk);
    }
  }

#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    pin_uniform(acc.a1[cb]);
    if (ROLE == kRoleKV) pin_uniform(acc.a2[cb]);
  }
  // the lane's own row token (q for kRoleQ, k for kRoleKV) for dx~ -> dx
  const uint16_t* tr = a.q + (bhN + (valid ? c.qi : 0)) * a.d;
  binarize_back_store<CB>(valid, tr, c.alpha, a.d, c.lh, ba.scale, acc.a1, ba.out1 + (bhN + (valid ? c.qi : 0)) * a.d);
  if (ROLE == kRoleKV && valid) {
    float* dvr = ba.out2 + (bhN + c.qi) * a.d;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c0 = cb * 32 + 8 * b + 4 * c.lh;
        const v4f o = {acc.a2[cb][4 * b], acc.a2[cb][4 * b + 1], acc.a2[cb][4 * b + 2], acc.a2[cb][4 * b + 3]};
        *reinterpret_cast<v4f*>(dvr + c0) = o;
      }
  }
}

template <int ROLE, int BIAS>
static int bwd_static_lds_for(int cb) {
  constexpr int kRed = kRedFloats * 4;
  switch (cb) {
    case 1: return 2 * sizeof(BwdTileBuf<ROLE, 1, 1, BIAS>) + kRed;
    case 2: return 2 * sizeof(BwdTileBuf<ROLE, 1, 2, BIAS>) + kRed;
    default: return 2 * sizeof(BwdTileBuf<ROLE, 2, 4, BIAS>) + kRed;
  }
}

int bwd_static_lds(int role, int dpad, int mode) {
  const int cb = dpad / 32;
  if (role == kRoleQ) {
    switch (mode) {
      case kBiasNone: return bwd_static_lds_for<kRoleQ, kBiasNone>(cb);
      case kBiasRows: return bwd_static_lds_for<kRoleQ, kBiasRows>(cb);
      default: return bwd_static_lds_for<kRoleQ, kBiasTable>(cb);
    }
  }
  switch (mode) {
    case kBiasNone: return bwd_static_lds_for<kRoleKV, kBiasNone>(cb);
    case kBiasRows: return bwd_static_lds_for<kRoleKV, kBiasRows>(cb);
    default: return bwd_static_lds_for<kRoleKV, kBiasTable>(cb);
  }
}

template <int ROLE, int NCH, int CB>
static int launch_bwd_nc(const BwdArgs& a, int mode, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.f.nwg), block(kThreads);
  const int lds = a.f.dyn_lds;
  switch (mode) {
    case kBiasNone:
      hipLaunchKernelGGL((attn_bwd_kernel<ROLE, NCH, CB, kBiasNone>), grid, block, lds, s, a);
      break;
    case kBiasRows:
      hipLaunchKernelGGL((attn_bwd_kernel<ROLE, NCH, CB, kBiasRows>), grid, block, lds, s, a);
      break;
    case kBiasTable:
      hipLaunchKernelGGL((attn_bwd_kernel<ROLE, NCH, CB, kBiasTable>), grid, block, lds, s, a);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_backward(const BwdArgs& a, int role, int mode, void* stream) {
  const int cb = a.f.dpad / 32;
  // the table gradient's wave windows hold two rows of 2gw - 1 entries
  // whenever a key tile spans two grid rows (window of two rows or more)
  if (role == kRoleQ && mode == kBiasRows && a.dtable &&
      (a.f.win_rows > 1 ? 2 : 1) * (2 * a.f.gw - 1) > kWaveWindow)
    return static_cast<int>(hipErrorInvalidValue);
  if (role == kRoleQ) {
    switch (cb) {
      case 1: return launch_bwd_nc<kRoleQ, 1, 1>(a, mode, stream);
      case 2: return launch_bwd_nc<kRoleQ, 1, 2>(a, mode, stream);
      case 4: return launch_bwd_nc<kRoleQ, 2, 4>(a, mode, stream);
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  }
  switch (cb) {
    case 1: return launch_bwd_nc<kRoleKV, 1, 1>(a, mode, stream);
    case 2: return launch_bwd_nc<kRoleKV, 1, 2>(a, mode, stream);
    case 4: return launch_bwd_nc<kRoleKV, 2, 4>(a, mode, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int fwd_table_lds(const FwdArgs& a, int mode) {
  if (mode == kBiasTable) return (2 * a.gh - 1) * (2 * a.gw - 1) * 4;
  return 0;
}

template <int BIAS>
static int static_lds_for(int cb) {
  constexpr int kRed = kRedFloats * 4;
  switch (cb) {
    case 1: return 2 * sizeof(TileBuf<1, 1, BIAS>) + kRed;
    case 2: return 2 * sizeof(TileBuf<1, 2, BIAS>) + kRed;
    case 3: return 2 * sizeof(TileBuf<2, 3, BIAS>) + kRed;
    case 4: return 2 * sizeof(TileBuf<2, 4, BIAS>) + kRed;
    case 5: return 2 * sizeof(TileBuf<3, 5, BIAS>) + kRed;
    case 6: return 2 * sizeof(TileBuf<3, 6, BIAS>) + kRed;
    case 7: return 2 * sizeof(TileBuf<4, 7, BIAS>) + kRed;
    default: return 2 * sizeof(TileBuf<4, 8, BIAS>) + kRed;
  }
}

int fwd_waves_per_simd(int dpad, int d) { return fwd_waves_for_blocks(dpad / 32 + (d % 32 == 0 ? 1 : 0), (d + 63) / 64); }

int fwd_static_lds(int dpad, int mode) {
  const int cb = dpad / 32;
  switch (mode) {
    case kBiasNone: return static_lds_for<kBiasNone>(cb);
    case kBiasRows: return static_lds_for<kBiasRows>(cb);
    case kBiasTable: return static_lds_for<kBiasTable>(cb);
    default: return static_lds_for<kBiasDense>(cb);
  }
}

template <int NCH, int CB, bool XONES>
static int launch_nc(const FwdArgs& a, int mode, void* stream) {
  const int lds = a.dyn_lds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.nwg), block(kThreads);
  switch (mode) {
    case kBiasNone:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, XONES, kBiasNone>), grid, block, lds, s, a);
      break;
    case kBiasRows:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, XONES, kBiasRows>), grid, block, lds, s, a);
      break;
    case kBiasDense:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, XONES, kBiasDense>), grid, block, lds, s, a);
      break;
    default:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, XONES, kBiasTable>), grid, block, lds, s, a);
      break;
  }
  return static_cast<int>(hipGetLastError());
}

template <int NCH, int CB>
static int launch_int8_nc(const FwdArgs& a, int mode, void* stream) {
  const int lds = a.dyn_lds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.nwg), block(kThreads);
  switch (mode) {
    case kBiasNone:
      hipLaunchKernelGGL((attn_fwd_int8_kernel<NCH, CB, kBiasNone>), grid, block, lds, s, a);
      break;
    case kBiasRows:
      hipLaunchKernelGGL((attn_fwd_int8_kernel<NCH, CB, kBiasRows>), grid, block, lds, s, a);
      break;
    case kBiasTable:
      hipLaunchKernelGGL((attn_fwd_int8_kernel<NCH, CB, kBiasTable>), grid, block, lds, s, a);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_attention_int8(const FwdArgs& a, int mode, void* stream) {
  switch (a.dpad / 32) {
    case 1: return launch_int8_nc<1, 1>(a, mode, stream);
    case 2: return launch_int8_nc<1, 2>(a, mode, stream);
    case 3: return launch_int8_nc<2, 3>(a, mode, stream);
    case 4: return launch_int8_nc<2, 4>(a, mode, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int launch_attention(const FwdArgs& a, int mode, void* stream) {
  const int cb = a.dpad / 32;
  const bool xones = (a.d % 32) == 0;
  switch (cb * 2 + (xones ? 1 : 0)) {
    case 2: return launch_nc<1, 1, false>(a, mode, stream);
    case 3: return launch_nc<1, 1, true>(a, mode, stream);
    case 4: return launch_nc<1, 2, false>(a, mode, stream);
    case 5: return launch_nc<1, 2, true>(a, mode, stream);
    case 6: return launch_nc<2, 3, false>(a, mode, stream);
    case 7: return launch_nc<2, 3, true>(a, mode, stream);
    case 8: return launch_nc<2, 4, false>(a, mode, stream);
    case 9: return launch_nc<2, 4, true>(a, mode, stream);
    case 10: return launch_nc<3, 5, false>(a, mode, stream);
    case 11: return launch_nc<3, 5, true>(a, mode, stream);
    case 12: return launch_nc<3, 6, false>(a, mode, stream);
    case 13: return launch_nc<3, 6, true>(a, mode, stream);
    case 14: return launch_nc<4, 7, false>(a, mode, stream);
    case 15: return launch_nc<4, 7, true>(a, mode, stream);
    case 16: return launch_nc<4, 8, false>(a, mode, stream);
    case 17: return launch_nc<4, 8, true>(a, mode, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace ba
