// Fused BinaryAttention forward for gfx950, pipelined across key blocks.
//
// Per (b, h) and query i it computes O_i = sum_j softmax_j(S_ij) V_j with
//   S_ij = scale * alpha_q,i * alpha_k,j * <sign q_i, sign k_j> + bias(h, i, j)
// (the scaled 1-bit similarity and the learnable bias of the BinaryAttention
// summaries: es page, section 2, "Representaciones Binarias Escaladas" and
// "Mejora mediante Sesgo"; ko page, section 2 (b)), tiled as FlashAttention2
// is (es page, section 2, "Implementacion en Hardware").
//
// Where the time goes on CDNA4.  A 32 x 32 block of scores costs a wave one
// fp4 MFMA for QK, 2d/16 bf16 MFMAs for P.V, one bf16 MFMA for the scale
// products w_ij = alpha_q,i alpha_k,j (scale log2e folded in; both factors
// enter as three bf16 terms, so w is exact to fp32 rounding), and per lane
// 16 scores of vector work: an FMA s w + bias, an exp2 and half a bf16 pack.
// The vector ALU is the scarcer unit (4 cycles per wave64 instruction, 8 for
// the exp2), so the kernel is built to keep it issuing:
//   * the QK product of the NEXT block is issued before this block's vector
//     work, so no wave waits on a matrix result (the S accumulator is double
//     buffered in registers);
//   * the P.V of the previous block (P and its V operands held in registers)
//     is issued at the start of the block and runs beside the vector work;
//   * the row sums l_i = sum_j P_ij come out of the matrix cores: one
//     v_mfma_f32_16x16x32_bf16 per 16 keys whose A operand is 1 where the
//     lane's B columns belong to the output row's query and 0 elsewhere, so
//     the product adds up exactly the bf16 P that multiplies V (no v_dot2,
//     which does not overlap with matrix instructions);
//   * V is read in its natural [key][channel] layout: the tile copies bring
//     contiguous key rows into LDS, and the transposing LDS read
//     (ds_read_b64_tr_b16) hands each lane 4 keys of one channel, which is
//     the A-operand layout of the P.V product; no transposed copy of V is
//     written anywhere.
//
// Workgroup: 4 waves x 32 queries = 128 queries of one (b, h).  Key tiles of
// 64 (two blocks of 32) go through three LDS buffers: tile t+2 is copied
// while tile t is computed and the QK of tile t+1's first block is issued;
// one barrier per tile, between its two blocks.
//
// Softmax in base 2 with log2(e) folded into the scales.  Every logit of the
// workgroup obeys |s| <= M = scale log2e max alpha_q max alpha_k d +
// log2e max|b|; when M <= 32 the softmax is taken with no offset (it does not
// depend on one), otherwise a running row maximum is kept and the
// accumulators are rescaled when it grows by more than 8.
#include "ba_internal.h"

namespace ba {

namespace {

constexpr float kFlashFastMax = 32.0f;

template <int D>
struct FDims {
  static_assert(D == 32 || D == 64 || D == 72 || D == 128, "the pipelined kernel takes d in {32, 64, 72, 128}");
  static constexpr int NCH = (D + 63) / 64;      // 64-channel fp4 QK chunks
  static constexpr int CB = (D + 31) / 32;        // 32-channel output blocks
  // d % 32 != 0: the V^T operand's channel d is 1 for every key, so output
  // channel d of P.V is the row sum and no row-sum product is needed
  static constexpr bool XONES = D % 32 != 0;
  static constexpr int PVS = CB + (XONES ? 0 : 1); // products per 16-key step
  static constexpr int ROW = 2 * D;               // bytes of one key's values
  static constexpr int VBYTES = 64 * ROW;         // V of one key tile
  static constexpr int VPIECES = (VBYTES + 1023) / 1024;  // 1 KiB copy pieces
  static constexpr int CPR = ROW / 16;            // 16-byte chunks per row
  static constexpr bool SWZ = (D & (D - 1)) == 0; // rows of a power-of-two size are swizzled
  static constexpr int KBYTES = NCH * 2048;       // fp4 key operands of one tile
  // floats of the table-row bias window of one tile (the host checks that
  // the grid's window fits)
  static constexpr int WIN = D <= 72 ? 1664 : 1152;
  static constexpr int WAVES = D <= 64 ? 3 : 2;   // waves per SIMD the registers allow
};

// Position of 16-byte chunk j of key row r of a V tile: j ^ vswz(r).  The
// transposing reads of one instruction cover 8 rows and 32 channels; with
// this swizzle those 512 bytes fall on every LDS bank exactly twice.  Rows
// of 144 bytes (d = 72) are not swizzled: 8 of them start 36 banks apart,
// which spreads them already.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return (D == 32 || !FDims<D>::SWZ) ? 0 : (D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3));
}

template <int D, int BIAS>
struct FBuf {
  v4i k[FDims<D>::NCH * 128];                  // fp4 key operands [chunk][key][half]
  uint32_t aks[192];                           // key scales as matrix operands: w0 w1 [64], w2 [64]
  v4u v[FDims<D>::VBYTES / 16];                // V rows, chunks swizzled
  // ones channel: channels d .. d+3 of every key = 1 0 0 0, then 4 zeros
  v4u vpad[FDims<D>::XONES ? 1 : 0];
  float win[BIAS == kBiasRows ? FDims<D>::WIN : 4];  // table-row bias window
};

template <int D>
struct FAcc {
  v16f o[FDims<D>::CB];  // O^T: lane = query, register = channel
  v4f l;                 // row sums (all four registers hold l of the lane's query;
                         // unused when the ones channel of O^T carries them)
};

// P.V of one finished block, waiting in registers for the next block.
template <int D>
struct FPend {
  uint32_t pk[8];                   // bf16 P: 16 keys x 2 steps of 16
  v8bf vop[2][FDims<D>::CB];        // V^T operands of the two steps
};

template <int D>
struct FCtx {
  const FwdArgs* a;
  int lane, wave, li, lh;
  int bh, head, q0, qi;
  float aq;                    // alpha_q * scale * log2e
  v4i qop[FDims<D>::NCH];      // the lane's query operand (fp4 +/-1)
  v8bf ones;                   // A operand of the row-sum product
  v8bf bq;                     // B operand of the scale product (the lane's aq split)
  int off_k, off_aks, off_win; // LDS byte offsets inside a buffer
  int off_v[FDims<D>::CB];     // byte offset of the lane's transposing reads
  // ones channel: full addresses of the last block's reads (read k of a
  // block takes rows 8 k .. 8 k + 7), pointing at the constant piece for
  // channels past d
  int off_vx[FDims<D>::XONES ? 8 : 1];
  int yq_lo;
  rsrc_t krs, ars, vrs, brs;   // sources of the tile copies
  uint32_t voff[FDims<D>::SWZ ? 1 : (FDims<D>::VPIECES + 3) / 4];  // the lane's byte offsets in its V pieces
  uint32_t vsn;                // bytes from one key's values to the next
  int win_bytes;
};

// The tile the copies fetch next: its first key and (table rows) the grid
// row and column of its first 32-key block.  gw % 32 == 0, so a block never
// straddles a grid row and the next block starts 32 columns on, or at
// column 0 of the next row.  Every field is wave-uniform.
struct FRun {
  int k0, by, bx;
};

// Left by the copy of a tile for the reads from its buffer: the uniform part
// of the bias-window offset of each of its two blocks.
struct FWin {
  int u[2];
};

template <typename T>
__device__ __forceinline__ T flds(const void* base, int byte_off) {
  return *reinterpret_cast<const T*>(__builtin_assume_aligned(static_cast<const char*>(base) + byte_off, 8));
}

// 4 keys of one channel from the natural V tile (see FCtx::off_v).
__device__ __forceinline__ v2u tr_read(const void* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<void*>(p)));
  return __builtin_bit_cast(v2u, r);
}

__device__ __forceinline__ v3f fmax3_block(float x, float y, float z, float* red) {
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

// ------------------------------------------------------------------ setup --
// The workgroup's (b, h) and query tile, LDS offsets and copy sources.
template <int D, int BIAS>
__device__ __forceinline__ void flash_index(FCtx<D>& c, const FwdArgs& a) {
  using F = FDims<D>;
  c.a = &a;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  c.li = c.lane & 31;
  c.lh = c.lane >> 5;
  int wg = blockIdx.x;
  if (a.xcd_remap) {
    // consecutive query tiles of a head on one XCD (its K/V stay in that L2)
    const int per = a.nwg >> 3;
    wg = (wg & 7) * per + (wg >> 3);
  }
  c.bh = wg / a.nqt;
  const int qt = wg - c.bh * a.nqt;
  c.head = c.bh % a.H;
  c.q0 = qt * kBM;
  c.qi = c.q0 + c.wave * 32 + c.li;

  const int b = c.bh / a.H;
  c.off_k = (c.li * 2 + c.lh) * 16;
  c.off_aks = c.li * 8;   // A row li of the scale product: key li of the block
  {
    // Transposing reads: in each group of 16 lanes, lane 4k + m supplies the
    // address of 4 channels of key row 4 lh + k, and lane i then receives
    // channel i of the group's 16 of those 4 rows.  Lane l (query column,
    // A row = channel 16 ((l/16) % 2) + i) thus gets keys 4 lh .. 4 lh + 3
    // of its channel: the slots 0..3 of its half of the 16-key step.
    const int g = c.lane >> 4, j = c.lane & 15, kk = j >> 2, m = j & 3;
    const int row = 4 * c.lh + kk;
#pragma unroll
    for (int cb = 0; cb < F::CB; ++cb) {
      const int ch0 = 32 * cb + 16 * (g & 1) + 4 * m;
      c.off_v[cb] = row * F::ROW + (((ch0 >> 3) ^ vswz<D>(row)) << 4) + ((ch0 >> 2) & 1) * 8;
    }
    if (F::XONES) {
      // the last block's channels past d come from the constant piece after
      // the tile (1 for channel d, 0 beyond), whatever the key row
      const int ch0 = 32 * (F::CB - 1) + 16 * (g & 1) + 4 * m;
      const int pad = F::VBYTES + (ch0 == D ? 0 : 8);
#pragma unroll
      for (int k = 0; k < 8; ++k) c.off_vx[k] = ch0 < D ? c.off_v[F::CB - 1] + 8 * k * F::ROW : pad;
    } else {
      c.off_vx[0] = 0;
    }
  }
  c.off_win = 0;
  c.yq_lo = 0;
  if (BIAS == kBiasRows) {
    // bias(i, j) = R[dy][gw-1-xi+xj], read from copy s = (gw-1-xi) & 3 at an
    // aligned float offset, in window row (yq - yq_lo) + (yk_hi - yk)
    const int yq = c.qi / a.gw, xq = c.qi - yq * a.gw;
    c.yq_lo = c.q0 / a.gw;
    const int bsel = (a.gw - 1 - xq) & 3;
    c.off_win = (((yq - c.yq_lo) * 4 + bsel) * a.Lpad + (a.gw - 1 - xq + 4 * c.lh - bsel)) * 4;
  }

  // copy sources: every range lies inside the section it names
  c.krs = make_rsrc(reinterpret_cast<const char*>(a.kop) + static_cast<int64_t>(c.bh) * (a.Npad / kBN) * F::KBYTES,
                    static_cast<uint32_t>((a.Npad / kBN) * F::KBYTES));
  c.ars = make_rsrc(a.aks + static_cast<int64_t>(c.bh) * (a.Npad / 64) * 192, static_cast<uint32_t>(a.Npad * 12));
  // V rows of this head; keys past N read as 0 (the range ends at key N-1)
  c.vsn = static_cast<uint32_t>(a.vs.sn * 2);
  c.vrs = make_rsrc(a.v + token_offset(a.vs, b, c.head, 0),
                    static_cast<uint32_t>((static_cast<int64_t>(a.N - 1) * a.vs.sn + D) * 2));
  // lane l of piece p copies 16-byte chunk e = 64 p + l of the tile: row
  // e / CPR, chunk e % CPR (read from the swizzled position, so that the
  // LDS copy, written in chunk order, holds each row swizzled).  Power-of-
  // two rows: the piece's first row goes in the scalar offset and voff[0]
  // serves every piece.
#pragma unroll
  for (int j = 0; j < (F::SWZ ? 1 : (F::VPIECES + 3) / 4); ++j) {
    const int e = F::SWZ ? c.lane : 64 * (c.wave + 4 * j) + c.lane, r = e / F::CPR, pos = e % F::CPR;
    c.voff[j] = static_cast<uint32_t>(r) * c.vsn + static_cast<uint32_t>((pos ^ vswz<D>(r)) << 4);
  }
  c.brs = c.ars;
  c.win_bytes = 0;
  if (BIAS == kBiasRows) {
    const int rows_p = 2 * a.gh - 1 + 2 * kBiasPadRows;
    c.brs = make_rsrc(a.bias4 + static_cast<int64_t>(c.head) * rows_p * 4 * a.Lpad,
                      static_cast<uint32_t>(rows_p * 16 * a.Lpad));
    c.win_bytes = a.win_rows * 16 * a.Lpad;
  }

}

// What the query side needs from global memory, loaded before the first
// tile copies are issued so that those stay in flight while it is used:
// the lane's 8-channel chunks of its query and the inputs of the logit bound.
template <int D>
struct FQin {
  uint4 q[FDims<D>::NCH][4];
  float km, bm;
};

template <int D, int BIAS>
__device__ __forceinline__ void flash_query_loads(const FCtx<D>& c, const FwdArgs& a, FQin<D>& in) {
  using F = FDims<D>;
  const int b = c.bh / a.H;
  const uint16_t* qrow = a.q + token_offset(a.qs, b, c.head, c.qi < a.N ? c.qi : 0);
#pragma unroll
  for (int ch = 0; ch < F::NCH; ++ch)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c0 = 32 * (2 * ch + c.lh) + 8 * k;
      in.q[ch][k] = make_uint4(0u, 0u, 0u, 0u);
      if (c.qi < a.N && c0 < D) in.q[ch][k] = *reinterpret_cast<const uint4*>(qrow + c0);
    }
  // one load per thread here, with no wait on it; the rest, for sequences
  // past 16384 keys or grids past 128 rows, in flash_queries
  const int tid = threadIdx.x, nblk = a.Npad / 64;
  in.km = tid < nblk ? a.kmax_blk[static_cast<int64_t>(c.bh) * nblk + tid] : 0.0f;
  in.bm = 0.0f;
  if (BIAS == kBiasRows) {
    const int rows = 2 * a.gh - 1;
    in.bm = tid < rows ? a.bias_row_max[c.head * rows + tid] : 0.0f;
  }
}

// The lane's packed query, its scale and operands, and the logit bound M
// (log2 units).
template <int D, int BIAS>
__device__ __forceinline__ float flash_queries(FCtx<D>& c, const FwdArgs& a, const FQin<D>& in, float* red) {
  using F = FDims<D>;
  // The lane's query: lane (li, lh) forms sign words 2 ch + lh of query qi
  // and the sum of |q| over them; the partner lane l ^ 32 holds the other
  // words, so the two partial sums give alpha_q = mean |q|.  Queries past N
  // are zero (scale 0).
  float qpart = 0.0f;
#pragma unroll
  for (int ch = 0; ch < F::NCH; ++ch) {
    const int word = 2 * ch + c.lh;
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (c.qi < a.N && 32 * word + 8 * k < D) {
        float part;
        w |= chunk_signs(in.q[ch][k], part) << (8 * k);
        qpart += part;
      }
    }
    c.qop[ch] = expand_signs_fp4(w, fp4_magnitude(word_valid(D, word)));
  }
  const float alpha_q = sum_halves(qpart) / static_cast<float>(D);
  c.aq = alpha_q * a.qscale;

  // Row-sum operand: lane l supplies A row l % 16 for k-slots 8 (l / 16) ..;
  // those slots hold P of query 16 ((l / 16) % 2) + column, so a 1 where
  // (l / 16) % 2 == ((l % 16) / 4) % 2 makes output row r sum the P of query
  // 16 ((r / 4) % 2) + column: every output register of lane l is l of its
  // query l % 32.
  {
    const bool one = ((c.lane >> 4) & 1) == (((c.lane & 15) >> 2) & 1);
    const __bf16 x = one ? (__bf16)1.0f : (__bf16)0.0f;
    c.ones = v8bf{x, x, x, x, x, x, x, x};
  }
  c.bq = __builtin_bit_cast(v8bf, scale_split_b(c.aq, c.lh == 0));

  float km = in.km, bm = in.bm;
  {
    const int tid = threadIdx.x, nblk = a.Npad / 64;
    for (int e = tid + kThreads; e < nblk; e += kThreads)
      km = fmaxf(km, a.kmax_blk[static_cast<int64_t>(c.bh) * nblk + e]);
    if (BIAS == kBiasRows) {
      const int rows = 2 * a.gh - 1;
      for (int e = tid + kThreads; e < rows; e += kThreads) bm = fmaxf(bm, a.bias_row_max[c.head * rows + e]);
    }
  }
  const v3f mx = fmax3_block(km, bm, alpha_q, red);
  return a.qscale * mx[2] * mx[0] * static_cast<float>(D) + mx[1];
}

// ---------------------------------------------------------------- copies --
// Starts the copies of the tile `run` names into `tb`, records its window
// offsets in `w` and advances `run` to the next tile.  Lane l of a wave
// fills bytes [16 l, 16 l + 16) of a 1 KiB piece (the 768 bytes of key-scale
// operands take 48 lanes of one wave).  Every source offset is uniform; the
// per-wave piece choices are uniform branches.
template <int D, int BIAS>
__device__ __forceinline__ void flash_copy(const FCtx<D>& c, FBuf<D, BIAS>& tb, FRun& run, FWin& w) {
  using F = FDims<D>;
  const FwdArgs& a = *c.a;
  // (the scalar offsets go through readfirstlane: the compiler cannot tell
  // that they are uniform and would otherwise loop over their lane values)
  const uint32_t k0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(run.k0));
  __builtin_assume(static_cast<unsigned>(c.wave) < 4u);  // kThreads = 256
  char* kdst = reinterpret_cast<char*>(&tb.k[0]);
#pragma unroll
  for (int j = 0; j < (2 * F::NCH + 3) / 4; ++j)
    if (c.wave + 4 * j < 2 * F::NCH)
      dma16(c.krs, kdst + (c.wave + 4 * j) * 1024, static_cast<uint32_t>(c.lane * 16),
            __builtin_amdgcn_readfirstlane(k0 / kBN * F::KBYTES + static_cast<uint32_t>((c.wave + 4 * j) * 1024)));
  char* vdst = reinterpret_cast<char*>(&tb.v[0]);
#pragma unroll
  for (int j = 0; j < (F::VPIECES + 3) / 4; ++j) {
    const int p = c.wave + 4 * j;
    // power-of-two rows: whole rows per piece, one lane offset for every
    // piece and the piece's first row in the scalar offset
    if (p < F::VPIECES)
      dma16(c.vrs, vdst + p * 1024, F::SWZ ? c.voff[0] : c.voff[j],
            __builtin_amdgcn_readfirstlane((k0 + static_cast<uint32_t>(F::SWZ ? p * (1024 / F::ROW) : 0)) * c.vsn));
  }
  if (c.wave == 3 && c.lane < 48)
    dma16(c.ars, &tb.aks[0], static_cast<uint32_t>(c.lane * 16), __builtin_amdgcn_readfirstlane(k0 * 12));
  run.k0 += kBN;
  if (BIAS == kBiasRows) {
    int ky[2], kx[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      ky[blk] = run.by;
      kx[blk] = run.bx;
      run.bx += 32;
      if (run.bx == a.gw) {
        run.bx = 0;
        run.by += 1;
      }
    }
    // window rows start at dy = yq_lo - yk_hi; yk_hi is the row of block 1
    const int dy0 = c.yq_lo - ky[1] + a.gh - 1 + kBiasPadRows;
    const uint32_t bs = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(dy0 * 16 * a.Lpad));
    // the lane's offset, formed here from the thread index: held across the
    // loop it would be one more register, which the allocator spills (and a
    // reload from scratch waits for every copy in flight)
    uint32_t tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const uint32_t loff = tid * 16;
    char* bdst = reinterpret_cast<char*>(&tb.win[0]);
    // 1 KiB pieces, every lane copying 16 bytes; when the window is not a
    // whole number of pieces its last piece ends at the window's end and
    // overlaps the one before it (both write the same bytes there), so no
    // copy depends on a lane condition.  Windows are at least 1280 bytes.
    const int full = c.win_bytes >> 10, pieces = (c.win_bytes + 1023) >> 10;
    const int back = c.win_bytes - 1024 * pieces;  // -(1024 - rest) or 0
#pragma unroll
    for (int j = 0; j < (F::WIN * 4 + 4095) / 4096; ++j) {
      const int p = c.wave + 4 * j;
      if (p < pieces) {
        const int sh = p == full ? back : 0;
        dma16(c.brs, bdst + p * 1024 + sh, loff + 4096 * j, bs + static_cast<uint32_t>(sh));
      }
    }
    w.u[0] = (ky[1] - ky[0]) * 16 * a.Lpad + kx[0] * 4;
    w.u[1] = kx[1] * 4;
  } else {
    w.u[0] = w.u[1] = 0;
  }
}

// --------------------------------------------------------------- compute --
// What a block reads from LDS before its first scores, fetched one block
// ahead: the A operand of its scale product and its first 4 bias values (the
// other 12 are read inside the block, a chunk or two ahead of their use).
struct FIn {
  v4u aop;       // scale_split_a of key li of the block (fourth word 0)
  v4f bias0;     // table rows: bias of the lane's scores 0..3 (0 without a table)
  int woff;      // table rows: the lane's window offset for the block
};

template <int D, int BIAS>
__device__ __forceinline__ void flash_fetch(const FCtx<D>& c, const FBuf<D, BIAS>& tb, const FWin& w, int blk,
                                            FIn& in) {
  const v2u w01 = flds<v2u>(tb.aks, c.off_aks + blk * 256);
  in.aop = v4u{w01[0], w01[1], flds<uint32_t>(tb.aks, 512 + c.off_aks / 2 + blk * 128), 0u};
  if (BIAS == kBiasRows) {
    int woff = c.off_win + w.u[blk];
    asm("" : "+v"(woff));  // one vector add here, the window reads take immediate offsets
    in.woff = woff;
    in.bias0 = flds<v4f>(tb.win, woff);
  } else {
    in.woff = 0;
    in.bias0 = v4f{};
  }
}

// fp4 key operands of block `blk`, one per 64-channel chunk.
template <int D, int BIAS>
__device__ __forceinline__ void flash_kops(const FCtx<D>& c, const FBuf<D, BIAS>& tb, int blk,
                                           v4i (&kop)[FDims<D>::NCH]) {
#pragma unroll
  for (int ch = 0; ch < FDims<D>::NCH; ++ch) kop[ch] = flds<v4i>(tb.k, c.off_k + ch * 2048 + blk * 1024);
}

// V^T operands of 16-key step `st` of block `blk` of the tile: per 32-channel
// block, two transposing reads (slots 0..3 and 4..7 of the lane's half).
template <int D, int BIAS>
__device__ __forceinline__ void flash_vops(const FCtx<D>& c, const FBuf<D, BIAS>& tb, int blk, int st,
                                           FPend<D>& pp) {
  using F = FDims<D>;
  const char* vb = reinterpret_cast<const char*>(&tb.v[0]);
#pragma unroll
  for (int cb = 0; cb < F::CB; ++cb) {
    int a_lo = c.off_v[cb] + (32 * blk + 16 * st) * F::ROW, a_hi = a_lo + 8 * F::ROW;
    if (F::XONES && cb == F::CB - 1) {
      a_lo = c.off_vx[4 * blk + 2 * st];
      a_hi = c.off_vx[4 * blk + 2 * st + 1];
    }
    const v2u lo = tr_read(vb + a_lo);
    const v2u hi = tr_read(vb + a_hi);
    pp.vop[st][cb] = __builtin_bit_cast(v8bf, v4u{lo[0], lo[1], hi[0], hi[1]});
  }
}

// Holds the next block's QK product where it is issued: left alone the
// compiler sinks it into the branch that runs the next block, right before
// the vector work that reads it, where the wave then waits for it.  The
// barrier keeps every instruction after this point after the product.
__device__ __forceinline__ void flash_qk_anchor(v16f& sn) {
  asm volatile("" : "+v"(sn));
  __builtin_amdgcn_sched_barrier(0);
}

// The scale products of the block whose A operand is `aop`: w[r] = aq of
// the lane's query times alpha_k of the key in accumulator register r (the
// QK layout), exact to fp32 rounding (see scale_split_a).
template <int D>
__device__ __forceinline__ v16f flash_scales(const FCtx<D>& c, const v4u& aop) {
  return mfma_bf16_32x32x16(__builtin_bit_cast(v8bf, aop), c.bq, v16f{});
}

// The matrix instructions of a block, in issue order: the pending block's
// first 16-key step (CB P.V products, then its row-sum product), the QK
// chunks of the next block, the pending block's second step.
template <int D>
struct FOrder {
  static constexpr int CB = FDims<D>::CB, NCH = FDims<D>::NCH, PVS = FDims<D>::PVS;
  static constexpr int NM = 2 * PVS + NCH;        // instructions per block
  static constexpr int QK0 = PVS;                 // first QK chunk
  static constexpr int QKL = PVS + NCH - 1;       // last QK chunk
  static constexpr int LASTV0 = CB - 1;           // last product reading step 0's V^T
  static constexpr int LASTV1 = PVS + NCH + CB - 1;  // last product reading step 1's V^T
};

template <int D>
__device__ __forceinline__ void flash_pv(int st, int i, const FCtx<D>& c, const FPend<D>& old, FAcc<D>& acc) {
  const v4u pw = {old.pk[4 * st], old.pk[4 * st + 1], old.pk[4 * st + 2], old.pk[4 * st + 3]};
  const v8bf p = __builtin_bit_cast(v8bf, pw);
  if (i < FDims<D>::CB)
    acc.o[i] = mfma_bf16_32x32x16(old.vop[st][i], p, acc.o[i]);
  else
    acc.l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.ones, p, acc.l, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void flash_mfma(int m, const FCtx<D>& c, const FPend<D>& old, const v4i (&kop)[FDims<D>::NCH],
                                           v16f& sn, FAcc<D>& acc) {
  using O = FOrder<D>;
  if (m < O::QK0) {
    flash_pv<D>(0, m, c, old, acc);
  } else if (m <= O::QKL) {
    const int ch = m - O::QK0;
    sn = mfma_signs_32x32x64(kop[ch], c.qop[ch], sn);
    if (m == O::QKL) flash_qk_anchor(sn);
  } else {
    flash_pv<D>(1, m - O::QKL - 1, c, old, acc);  // m - QKL - 1 < PVS
  }
}

// One block, offset-free softmax.  The pending block's matrix work and the
// next block's QK are spread over four chunks of vector work (4 scores
// each), so that no wave issues its matrix instructions back to back and the
// vector ALU keeps issuing beside them; scheduling barriers hold that order.
// The scores are s w + bias with the block's scale products w; after the
// last chunk w takes the next block's (its A operand in innext).  Writes P
// of this block into nw.pk and its V^T operands into nw.vop, each step's
// once the pending block's products have consumed the same registers' old
// values.
template <int D, int BIAS>
__device__ __forceinline__ void flash_block_fast(const FCtx<D>& c, const FBuf<D, BIAS>& tb, int blk, const v16f& s,
                                                 const FIn& in, const v4i (&kop)[FDims<D>::NCH], v16f& sn,
                                                 const FPend<D>& old, FPend<D>& nw, FAcc<D>& acc, int key0,
                                                 bool mask, v16f& w, const FIn& innext) {
  using O = FOrder<D>;
  constexpr int NM = O::NM;
  const FwdArgs& a = *c.a;
  v4f bias[4];
  bias[0] = in.bias0;
  bias[1] = bias[2] = bias[3] = v4f{};
  if (BIAS == kBiasRows) {
    bias[1] = flds<v4f>(tb.win, in.woff + 32);
    bias[2] = flds<v4f>(tb.win, in.woff + 64);
  }
  sn = v16f{};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int m = b * NM / 4; m < (b + 1) * NM / 4; ++m) flash_mfma<D>(m, c, old, kop, sn, acc);
    if (b * NM / 4 <= O::LASTV0 && O::LASTV0 < (b + 1) * NM / 4) flash_vops(c, tb, blk, 0, nw);
    if (b * NM / 4 <= O::LASTV1 && O::LASTV1 < (b + 1) * NM / 4) flash_vops(c, tb, blk, 1, nw);
    if (b == 0 && BIAS == kBiasRows) bias[3] = flds<v4f>(tb.win, in.woff + 96);
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = BIAS == kBiasRows ? fmaf(s[4 * b + e], w[4 * b + e], bias[b][e]) : s[4 * b + e] * w[4 * b + e];
    if (BIAS != kBiasRows && mask) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key0 + 8 * b + 4 * c.lh + e >= a.N) x[e] = -INFINITY;
    }
    nw.pk[2 * b] = pack_bf16x2(fast_exp2(x[0]), fast_exp2(x[1]));
    nw.pk[2 * b + 1] = pack_bf16x2(fast_exp2(x[2]), fast_exp2(x[3]));
    // keep this chunk's vector work here: left alone, the compiler sinks it
    // to the product that uses it, past the barrier and into the next block
    asm volatile("" : "+v"(nw.pk[2 * b]), "+v"(nw.pk[2 * b + 1]));
    __builtin_amdgcn_sched_barrier(0);
  }
  w = flash_scales(c, innext.aop);
}

// One block with the online softmax: the pending block's products and the
// next block's QK go first (a rescale of the accumulators must cover the
// products), then the logits s w + bias, the row maximum (log2 units, mrow)
// with the lazy rescale, P = exp2(s - mrow), and the next block's scale
// products.
template <int D, int BIAS>
__device__ __forceinline__ void flash_block_exact(const FCtx<D>& c, const FBuf<D, BIAS>& tb, int blk,
                                                  const v16f& s, const FIn& in,
                                                  const v4i (&kop)[FDims<D>::NCH], v16f& sn,
                                                  const FPend<D>& old, FPend<D>& nw, FAcc<D>& acc, int key0,
                                                  bool mask, float& mrow, v16f& w, const FIn& innext) {
  const FwdArgs& a = *c.a;
  v4f bias[4];
  bias[0] = in.bias0;
#pragma unroll
  for (int b = 1; b < 4; ++b) bias[b] = BIAS == kBiasRows ? flds<v4f>(tb.win, in.woff + 32 * b) : v4f{};
  sn = v16f{};
#pragma unroll
  for (int m = 0; m < FOrder<D>::NM; ++m) flash_mfma<D>(m, c, old, kop, sn, acc);
  flash_vops(c, tb, blk, 0, nw);
  flash_vops(c, tb, blk, 1, nw);
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    x[r] = BIAS == kBiasRows ? fmaf(s[r], w[r], bias[r >> 2][r & 3]) : s[r] * w[r];
  if (BIAS != kBiasRows && mask) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + 8 * (r >> 2) + 4 * c.lh + (r & 3) >= a.N) x[r] = -INFINITY;
  }
  float mt = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
  mt = max_halves(mt);
  const float mnew = fmaxf(mrow, mt);
  if (__any(mnew > mrow + 8.0f)) {
    // a row that has seen only -inf logits keeps its (zero) sums
    const float f = mnew > -INFINITY ? fast_exp2(mrow - mnew) : 1.0f;
#pragma unroll
    for (int cb = 0; cb < FDims<D>::CB; ++cb) acc.o[cb] *= f;
    acc.l *= f;
    mrow = mnew;
  }
  // such a row takes its P against 0: exp2(-inf) = 0, not exp2(-inf + inf)
  const float off = mrow > -INFINITY ? mrow : 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) nw.pk[j] = pack_bf16x2(fast_exp2(x[2 * j] - off), fast_exp2(x[2 * j + 1] - off));
  w = flash_scales(c, innext.aop);
}

template <int D, int BIAS, bool EXACT>
__device__ __forceinline__ void flash_block(const FCtx<D>& c, const FBuf<D, BIAS>& tb, int blk, const v16f& s,
                                            const FIn& in, const v4i (&kop)[FDims<D>::NCH], v16f& sn,
                                            const FPend<D>& old, FPend<D>& nw, FAcc<D>& acc, int key0, bool mask,
                                            float& mrow, v16f& w, const FIn& innext) {
  if (EXACT)
    flash_block_exact<D, BIAS>(c, tb, blk, s, in, kop, sn, old, nw, acc, key0, mask, mrow, w, innext);
  else
    flash_block_fast<D, BIAS>(c, tb, blk, s, in, kop, sn, old, nw, acc, key0, mask, w, innext);
}

// Wave priority (when the host sets prio_balance: every workgroup of the
// grid is resident at once).  Equal-priority waves issue oldest first, so
// left alone the first workgroup of a CU finishes long before the last one;
// instead the priority steps down from 3 to 0 at 5/8, 6/8 and 7/8 of the key
// tiles, so that waves that get there first yield to the others.  The
// thresholds th[] are tile indices; the step is taken on the tile that
// reaches one.
struct FPrio {
  int th[3];  // first tile of priority 2, 1, 0 (past the last tile: never)
  int level;
};

__device__ __forceinline__ void flash_priority(FPrio& p, int t) {
  const int want = t >= p.th[2] ? 0 : (t >= p.th[1] ? 1 : (t >= p.th[0] ? 2 : 3));
  if (__builtin_expect(want != p.level, 0)) {
    p.level = want;
    if (want == 2)
      __builtin_amdgcn_s_setprio(2);
    else if (want == 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  }
}

// One key tile: block 0, the barrier, the copies of the tile `run` names
// (t+2), block 1.  On entry s0 / in0 hold the QK and the LDS inputs of this
// tile's block 0 and ppa the pending block; on exit the same for the next
// tile.  Block 1's QK and inputs go through s1 / in1, its pending block
// through ppb.  wc, wn, wf: the window offsets of the tiles in cur, nxt and
// far.  INNER: a tile with a copy to issue and two full blocks (every tile
// but the last four), so none of the per-tile tests run.
template <int D, int BIAS, bool EXACT, bool INNER>
__device__ __forceinline__ void flash_tile(const FCtx<D>& c, const FBuf<D, BIAS>& cur, const FBuf<D, BIAS>& nxt,
                                           FBuf<D, BIAS>& far, const FWin& wc, const FWin& wn, FWin& wf, FRun& run,
                                           FPrio& prio, int t, int nkt, v16f& s0, v16f& s1, FIn& in0, FIn& in1,
                                           FPend<D>& ppa, FPend<D>& ppb, FAcc<D>& acc, float& mrow, v16f& w) {
  const FwdArgs& a = *c.a;
  const int k0 = t * kBN;
  const bool has1 = INNER || k0 + 32 < a.N;
  v4i kop[FDims<D>::NCH];
  // block 0: the next block is this tile's block 1
  flash_kops(c, cur, 1, kop);
  flash_fetch(c, cur, wc, 1, in1);
  flash_block<D, BIAS, EXACT>(c, cur, 0, s0, in0, kop, s1, ppa, ppb, acc, k0, !INNER && k0 + 32 > a.N, mrow, w,
                              in1);
  // tile t+1 is in `nxt` once every wave's copies have landed; every wave is
  // done with tile t-1, whose buffer `far` takes tile t+2
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (INNER || t + 2 < nkt) flash_copy(c, far, run, wf);
  flash_priority(prio, t);
  if (__builtin_expect(has1, 1)) {
    // block 1: the next block is tile t+1's block 0
    flash_kops(c, nxt, 0, kop);
    flash_fetch(c, nxt, wn, 0, in0);
    flash_block<D, BIAS, EXACT>(c, cur, 1, s1, in1, kop, s0, ppb, ppa, acc, k0 + 32, !INNER && k0 + 64 > a.N, mrow,
                                w, in0);
  } else {
    ppa = ppb;  // the last tile ends after block 0
  }
}

// All keys, after the copies of tiles 0 and 1 into b0 and b1 (run names
// tile 2; w0, w1 hold the window offsets of tiles 0 and 1); returns the
// offset the sums are taken against (log2 units).
template <int D, int BIAS, bool EXACT>
__device__ __forceinline__ float flash_pass(const FCtx<D>& c, FBuf<D, BIAS>& b0, FBuf<D, BIAS>& b1,
                                            FBuf<D, BIAS>& b2, FAcc<D>& acc, FRun run, FWin w0, FWin w1) {
  const FwdArgs& a = *c.a;
#pragma unroll
  for (int cb = 0; cb < FDims<D>::CB; ++cb) acc.o[cb] = v16f{};
  acc.l = v4f{};
  float mrow = EXACT ? -INFINITY : 0.0f;
  const int nkt = (a.N + kBN - 1) / kBN;
  FPrio prio;
  prio.level = 3;
  for (int i = 0; i < 3; ++i) prio.th[i] = a.prio_balance ? ((5 + i) * nkt + 7) / 8 : nkt;
  if (a.prio_balance) __builtin_amdgcn_s_setprio(3);
  FWin w2;
  w2.u[0] = w2.u[1] = 0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v16f s0, s1 = v16f{};
  {
    v4i kop[FDims<D>::NCH];
    flash_kops(c, b0, 0, kop);
    s0 = v16f{};
#pragma unroll
    for (int ch = 0; ch < FDims<D>::NCH; ++ch) s0 = mfma_signs_32x32x64(kop[ch], c.qop[ch], s0);
  }
  FIn in0, in1;
  flash_fetch(c, b0, w0, 0, in0);
  v16f wk = flash_scales(c, in0.aop);  // the scale products of block 0
  // nothing is pending before the first block: P = 0
  FPend<D> ppa, ppb;
#pragma unroll
  for (int j = 0; j < 8; ++j) ppa.pk[j] = 0u;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int cb = 0; cb < FDims<D>::CB; ++cb) ppa.vop[st][cb] = v8bf{};
  // Inner tiles (a copy to issue and two full blocks; every tile but the
  // last four) in groups of three with no per-tile tests, then the rest.
  int t = 0;
  for (; t + 5 <= nkt; t += 3) {
    flash_tile<D, BIAS, EXACT, true>(c, b0, b1, b2, w0, w1, w2, run, prio, t, nkt, s0, s1, in0, in1, ppa, ppb, acc,
                                     mrow, wk);
    flash_tile<D, BIAS, EXACT, true>(c, b1, b2, b0, w1, w2, w0, run, prio, t + 1, nkt, s0, s1, in0, in1, ppa, ppb, acc,
                                     mrow, wk);
    flash_tile<D, BIAS, EXACT, true>(c, b2, b0, b1, w2, w0, w1, run, prio, t + 2, nkt, s0, s1, in0, in1, ppa, ppb, acc,
                                     mrow, wk);
  }
  for (; t < nkt; t += 3) {
    flash_tile<D, BIAS, EXACT, false>(c, b0, b1, b2, w0, w1, w2, run, prio, t, nkt, s0, s1, in0, in1, ppa, ppb, acc,
                                      mrow, wk);
    if (t + 1 >= nkt) break;
    flash_tile<D, BIAS, EXACT, false>(c, b1, b2, b0, w1, w2, w0, run, prio, t + 1, nkt, s0, s1, in0, in1, ppa, ppb,
                                      acc, mrow, wk);
    if (t + 2 >= nkt) break;
    flash_tile<D, BIAS, EXACT, false>(c, b2, b0, b1, w2, w0, w1, run, prio, t + 2, nkt, s0, s1, in0, in1, ppa, ppb,
                                      acc, mrow, wk);
  }
  // drain: the last block's P.V and row sums
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < FDims<D>::PVS; ++i) flash_pv<D>(st, i, c, ppa, acc);
  return mrow;
}

// O = O^T / l in bf16; each wave stages its 32 rows in LDS (the V regions of
// two buffers, free after the key loop) and writes whole rows with
// nontemporal 16-byte stores.
template <int D>
__device__ __forceinline__ void flash_epilogue(const FCtx<D>& c, const FwdArgs& a, FAcc<D>& acc, float mrow,
                                               unsigned char* stage0, unsigned char* stage1) {
  using F = FDims<D>;
#pragma unroll
  for (int cb = 0; cb < F::CB; ++cb) pin_uniform(acc.o[cb]);
  float l = acc.l[0];
  if (F::XONES) {
    // output channel d: block CB-1, register 4 (ch / 8) + ch % 4 of the lanes
    // of half (ch / 4) % 2, ch = d - 32 (CB-1)
    constexpr int ch = D - 32 * (F::CB - 1), r = 4 * (ch / 8) + ch % 4, half = (ch / 4) % 2;
    l = __shfl(acc.o[F::CB - 1][r], c.li + 32 * half, 64);
  }
  {
    float e = l;
    asm volatile("" : "+v"(e));
    l = e;
  }
  const float inv = 1.0f / l;
  if (a.lse_out && c.lh == 0 && c.qi < a.N)
    a.lse_out[static_cast<int64_t>(c.bh) * a.N + c.qi] = (mrow + log2f(l)) * kLn2;
  constexpr int C = D / 8;
  constexpr int sw = (C & 7) == 0 ? 7 : 0;
  unsigned char* ws = (c.wave < 2 ? stage0 : stage1) + (c.wave & 1) * 64 * D;
  __syncthreads();  // every wave is past its last read of the tile buffers
#pragma unroll
  for (int cb = 0; cb < FDims<D>::CB; ++cb)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c0 = cb * 32 + 8 * b + 4 * c.lh;
      if (c0 >= D) continue;  // padded channels (the ones channel among them)
      v2u w;
      w[0] = pack_bf16x2(acc.o[cb][4 * b + 0] * inv, acc.o[cb][4 * b + 1] * inv);
      w[1] = pack_bf16x2(acc.o[cb][4 * b + 2] * inv, acc.o[cb][4 * b + 3] * inv);
      *reinterpret_cast<v2u*>(ws + (c.li * C + ((c0 >> 3) ^ (c.li & sw))) * 16 + (c0 & 4) * 2) = w;
    }
  __syncthreads();
  const int r0 = c.q0 + c.wave * 32;
  const int64_t b = c.bh / a.H;
  for (int e = c.lane; e < 32 * C; e += 64) {
    const int r = e / C, j = e - r * C;
    if (r0 + r < a.N) {
      const v4u x = flds<v4u>(ws, (r * C + (j ^ (r & sw))) * 16);
      __builtin_nontemporal_store(x, reinterpret_cast<v4u*>(a.o + token_offset(a.os, b, c.head, r0 + r) + 8 * j));
    }
  }
}

template <int D, int BIAS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FDims<D>::WAVES)))
flash_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) FBuf<D, BIAS> b0;
  __shared__ __attribute__((aligned(16))) FBuf<D, BIAS> b1;
  __shared__ __attribute__((aligned(16))) FBuf<D, BIAS> b2;
  FCtx<D> c;
  flash_index<D, BIAS>(c, a);
  // The query side's global loads go out first and the copies of tiles 0
  // and 1 after them, so that the copies are still in flight while the
  // queries are packed and the logit bound is reduced.
  FQin<D> qin;
  flash_query_loads<D, BIAS>(c, a, qin);
  FRun run;
  run.k0 = 0;
  run.by = 0;
  run.bx = 0;
  FWin w0, w1;
  flash_copy(c, b0, run, w0);
  w1.u[0] = w1.u[1] = 0;
  if (a.N > kBN) flash_copy(c, b1, run, w1);
  if (FDims<D>::XONES && threadIdx.x < 3) {
    // the constant piece of each buffer (the first barrier of the key loop
    // orders these writes before every read)
    FBuf<D, BIAS>& pb = threadIdx.x == 0 ? b0 : (threadIdx.x == 1 ? b1 : b2);
    pb.vpad[0] = v4u{0x3f80u, 0u, 0u, 0u};
  }
  // the bound's reduction borrows b2, which the first copies leave alone
  // (it takes tile 2, after several barriers)
  const float M = flash_queries<D, BIAS>(c, a, qin, reinterpret_cast<float*>(&b2.v[0]));
  FAcc<D> acc;
  float mrow;
  if (M <= kFlashFastMax)  // false for NaN as well
    mrow = flash_pass<D, BIAS, false>(c, b0, b1, b2, acc, run, w0, w1);
  else
    mrow = flash_pass<D, BIAS, true>(c, b0, b1, b2, acc, run, w0, w1);
  flash_epilogue<D>(c, a, acc, mrow, reinterpret_cast<unsigned char*>(&b0.v[0]),
                    reinterpret_cast<unsigned char*>(&b1.v[0]));
}

template <int D, int BIAS>
int flash_lds() {
  return static_cast<int>(3 * sizeof(FBuf<D, BIAS>));
}

template <int D>
int launch_flash_d(const FwdArgs& a, int mode, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.nwg), block(kThreads);
  if (mode == kBiasRows)
    hipLaunchKernelGGL((flash_fwd_kernel<D, kBiasRows>), grid, block, a.dyn_lds, s, a);
  else
    hipLaunchKernelGGL((flash_fwd_kernel<D, kBiasNone>), grid, block, a.dyn_lds, s, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

bool flash_supported(int d, int mode, int win_rows, int Lpad) {
  if (d != 32 && d != 64 && d != 72 && d != 128) return false;
  if (mode == kBiasNone) return true;
  if (mode != kBiasRows) return false;
  const int win = win_rows * 4 * Lpad;
  // the copies take the window in 1 KiB pieces, the last one ending at the
  // window's end
  return win >= 256 && win <= (d <= 72 ? FDims<64>::WIN : FDims<128>::WIN);
}

int flash_static_lds(int d, int mode) {
  const bool rows = mode == kBiasRows;
  switch (d) {
    case 32: return rows ? flash_lds<32, kBiasRows>() : flash_lds<32, kBiasNone>();
    case 64: return rows ? flash_lds<64, kBiasRows>() : flash_lds<64, kBiasNone>();
    case 72: return rows ? flash_lds<72, kBiasRows>() : flash_lds<72, kBiasNone>();
    default: return rows ? flash_lds<128, kBiasRows>() : flash_lds<128, kBiasNone>();
  }
}

int flash_waves_per_simd(int d) { return d <= 64 ? FDims<64>::WAVES : FDims<128>::WAVES; }
static_assert(FDims<72>::WAVES == FDims<128>::WAVES, "d = 72 takes the d = 128 budget");

int launch_flash(const FwdArgs& a, int mode, void* stream) {
  switch (a.d) {
    case 32: return launch_flash_d<32>(a, mode, stream);
    case 64: return launch_flash_d<64>(a, mode, stream);
    case 72: return launch_flash_d<72>(a, mode, stream);
    case 128: return launch_flash_d<128>(a, mode, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace ba
