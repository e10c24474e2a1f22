// Prologue kernel of the BinaryAttention forward, plus the standalone sign
// pack.
//
// One launch runs up to three independent jobs, split by block index:
//   * pack (ba_pack_signs): per token of one tensor, the scale alpha =
//     mean |x| over d and the packed sign words (s_i = mu sign(q_i),
//     "Representaciones Binarias Escaladas" of the BinaryAttention summary).
//   * kv (the forward): per 64-token tile of one (b, h), the key scales and
//     their tile maximum, the key signs as the fp4 +/-1 operand tile the
//     fused kernel copies straight into LDS, and a key-major copy of the
//     value tile (V^T) whose keys are permuted inside each group of 16 into
//     the P.V operand order.  The queries are packed by the fused kernel.
//   * bias rows: the relative-position table ("Mejora mediante Sesgo") as
//     float32 * log2(e), with the dx axis reversed, in four copies shifted
//     by 0..3 entries, so that any 4 consecutive entries can be read with
//     one aligned 16-byte LDS load.
// All three are bound by HBM traffic.  Loads are 16-byte and coalesced, and
// each thread issues all of its loads before it uses any of them.
#include "ba_internal.h"

namespace ba {

namespace {

// At most this many 16-byte chunks of one tensor per thread and tile
// (64 tokens x d/8 chunks, d <= 256).
constexpr int kMaxChunks = kPackTok * 32 / kThreads;

// Sum of the C chunk partials of one token (row of 33 floats), pairwise in a
// fixed order: deterministic, within a few ulps of the exact sum for d <= 256.
// 16 bytes that this launch writes and only the next one reads: a
// nontemporal store, which leaves the line to stream out to memory now
// instead of staying dirty in L2 until the end-of-kernel writeback (about
// 2 us less per forward at N = 4096 with the table).
template <typename T>
__device__ __forceinline__ void stream_out(T* dst, v4u x) {
  __builtin_nontemporal_store(x, reinterpret_cast<v4u*>(dst));
}

__device__ __forceinline__ float token_sum(float* v, int C) {
  for (int s = 1; s < C; s *= 2)
    for (int i = 0; i + s < C; i += 2 * s) v[i] += v[i + s];
  return v[0];
}

// The sign words of a 64-token block in LDS, as bytes: channel 8*ch + b ->
// word ch/4, bit 8*(ch%4) + b, i.e. byte ch of the token's little-endian word
// array.  Chunks past d give zero bytes.
__device__ __forceinline__ void store_sign_bytes(unsigned char* sb, int tok, int ch, int W, uint32_t byte) {
  sb[tok * 4 * W + ch] = static_cast<unsigned char>(byte);
}
__device__ __forceinline__ void zero_pad_bytes(unsigned char* sb, int C, int W) {
  const int pad = 4 * W - C;
  for (int e = threadIdx.x; e < kPackTok * pad; e += kThreads) {
    const int tok = e / pad;
    sb[tok * 4 * W + C + (e - tok * pad)] = 0;
  }
}

}  // namespace

int prologue_lds(int d, bool kv) {
  const int W = (d + 31) / 32;
  const int common = kPackTok * 33 * 4 + kPackTok * W * 4;  // partial sums, sign words
  // + the value tile and, for the 8-bit value codes, 1/scale per channel
  return kv ? common + kPackTok * (d + 8) * 2 + 32 * W * 4 : common;
}

// ---------------------------------------------------------------- pack ----
// One block = 64 consecutive tokens of the flattened [BH*N] token list.
__device__ void pack_block(const PackJob& job, int64_t blk, unsigned char* smem) {
  const int d = job.d, W = job.W, C = d / 8;
  const int64_t T = job.BH * static_cast<int64_t>(job.N);
  const int64_t t0 = blk * kPackTok;
  float* sp = reinterpret_cast<float*>(smem);                          // [64][33]
  unsigned char* sb = smem + kPackTok * 33 * 4;                         // [64][4W]
  const int total = static_cast<int>(T - t0 < kPackTok ? (T - t0) * C : kPackTok * C);
  const uint16_t* base = job.x + t0 * d;
  uint4 raw[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int g = threadIdx.x + i * kThreads;
    raw[i] = make_uint4(0u, 0u, 0u, 0u);
    if (g < total) raw[i] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(g) * 8);
  }
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int g = threadIdx.x + i * kThreads;
    if (g < kPackTok * C) {
      const int tok = g / C, ch = g - tok * C;
      float part;
      store_sign_bytes(sb, tok, ch, W, chunk_signs(raw[i], part));
      sp[tok * 33 + ch] = part;
    }
  }
  zero_pad_bytes(sb, C, W);
  __syncthreads();
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(sb);
  for (int e = threadIdx.x; e < kPackTok * W; e += kThreads) {
    const int64_t t = t0 + e / W;
    if (t < T) job.bits[t0 * W + e] = sw[e];
  }
  if (threadIdx.x < kPackTok) {
    const int64_t t = t0 + threadIdx.x;
    const float sum = token_sum(sp + threadIdx.x * 33, C);
    if (t < T) job.alpha[t] = sum / static_cast<float>(d);
  }
}

// ------------------------------------------------------------------ kv ----
// The V^T tile is written as one contiguous dpad x 128-byte block, in the
// order the fused kernel copies straight into LDS:
//   * rows c < d hold V[.., c]; rows d and d+4 (d % 32 != 0) hold 1.0 for
//     every key < N, so the P.V product also yields the row sums of P; the
//     other rows are 0;
//   * keys are permuted inside each group of 16 into the P.V slot order
//     (slots 8h..8h+3 = keys 4h..4h+3, slots 8h+4..8h+7 = keys 8+4h..8+4h+3);
//   * the eight 16-byte chunks of row c are stored at chunk position
//     q ^ ((c >> 1) & 7), so that 16 lanes reading one chunk from 16
//     consecutive rows touch 16 different 4-bank groups.
__device__ __forceinline__ int vt_slot_key(int slot) {
  const int g = slot >> 4, s16 = slot & 15, hh = s16 >> 3, s = s16 & 7;
  return g * 16 + (s < 4 ? 4 * hh + s : 8 + 4 * hh + (s - 4));
}


__device__ void kv_codes(const KvJob& job, int64_t blk, int64_t bh, int tile, const uint16_t* vs, int stride,
                         float* sinv, float* red);

// KONLY: the keys alone (no value tile, codes, maxima or sign tiles), the
// variant the forward launches when its fused kernel reads V in place.
template <bool KONLY>
__device__ void kv_block(const KvJob& job, int64_t blk, unsigned char* smem) {
  const int d = job.d, W = job.W, C = d / 8, stride = d + 8;  // bf16 units
  const int tiles = job.Npad / kPackTok;
  const int64_t bh = blk / tiles;
  const int tile = static_cast<int>(blk - bh * tiles), n0 = tile * kPackTok;
  float* sp = reinterpret_cast<float*>(smem);                              // [64][33]
  unsigned char* sb = smem + kPackTok * 33 * 4;                             // [64][4W]
  uint16_t* vs = reinterpret_cast<uint16_t*>(sb + kPackTok * 4 * W);       // [64][d+8]

  // Chunk g of the tile is token n0 + g / C, channels 8 (g % C) .. + 7; a
  // token's channels are contiguous, tokens are ks.sn / vs.sn apart.  Tokens
  // past N read as 0.
  const int rows = job.N - n0 < kPackTok ? job.N - n0 : kPackTok;
  const int total = rows * C;
  const int64_t b = bh / job.H, h = bh - b * job.H;
  const uint16_t* kbase = job.k + token_offset(job.ks, b, h, n0);
  const uint16_t* vbase = job.v + token_offset(job.vs, b, h, n0);
  // the values are read only for an output that needs them
  const bool want_v = !KONLY && (job.vt || job.vq || job.vmax || job.vnat);
  uint4 kr[kMaxChunks], vr[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int g = threadIdx.x + i * kThreads;
    kr[i] = vr[i] = make_uint4(0u, 0u, 0u, 0u);
    if (g < total) {
      const int tok = g / C, ch = g - tok * C;
      kr[i] = *reinterpret_cast<const uint4*>(kbase + tok * job.ks.sn + ch * 8);
      if (want_v) vr[i] = *reinterpret_cast<const uint4*>(vbase + tok * job.vs.sn + ch * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int g = threadIdx.x + i * kThreads;
    if (g < kPackTok * C) {
      const int tok = g / C, ch = g - tok * C;
      float part;
      store_sign_bytes(sb, tok, ch, W, chunk_signs(kr[i], part));
      sp[tok * 33 + ch] = part;
      if (!KONLY && (job.vt || job.vq)) *reinterpret_cast<uint4*>(vs + tok * stride + ch * 8) = vr[i];
      if (!KONLY && job.vnat)
        stream_out(job.vnat + (bh * job.Npad + n0 + tok) * d + ch * 8, v4u{vr[i].x, vr[i].y, vr[i].z, vr[i].w});
    }
  }
  zero_pad_bytes(sb, C, W);
  __shared__ float vwave[kThreads / 64];
  if (!KONLY && job.vmax) {
    // largest |v| of the tile (chunks past N hold 0)
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(static_cast<uint16_t>(w[e] & 0xffffu))),
                           fabsf(bf16_to_f32(static_cast<uint16_t>(w[e] >> 16)))));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) vwave[threadIdx.x >> 6] = m;
  }
  __syncthreads();
  if (!KONLY && job.vmax && threadIdx.x == 0) {
    float m = vwave[0];
    for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, vwave[i]);
    job.vmax[blk] = m;
  }

  // key scales and the tile's largest one (wave 0 holds all 64 tokens)
  if (threadIdx.x < kPackTok) {
    const int tok = threadIdx.x;
    const float a = tok < rows ? token_sum(sp + tok * 33, C) / static_cast<float>(d) : 0.0f;
    if (job.alpha) job.alpha[bh * job.Npad + n0 + tok] = a;
    if (job.aks) {
      uint32_t w[3];
      scale_split_a(a, w);
      uint32_t* t = job.aks + blk * 192;
      *reinterpret_cast<v2u*>(t + 2 * tok) = v2u{w[0], w[1]};
      t[128 + tok] = w[2];
    }
    float m = a;  // scales are >= 0
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (tok == 0) job.alpha_max[blk] = m;
  }

  // fp4 operands: [chunk][key][half][4 dwords], word 2*chunk + half of the
  // key, expanded exactly as the fused kernel expands its query words.
  // Consecutive threads write consecutive 16-byte pieces.
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(sb);
  uint4* kdst = reinterpret_cast<uint4*>(job.kop) + blk * (kPackTok * 2 * job.nch);
  for (int e = threadIdx.x; e < kPackTok * 2 * job.nch; e += kThreads) {
    const int ch = e >> 7, key = (e >> 1) & (kPackTok - 1), w = 2 * ch + (e & 1);
    const uint32_t word = w < W ? sw[key * W + w] : 0u;
    const v4i op = expand_signs_fp4(word, fp4_magnitude(word_valid(d, w)));
    stream_out(kdst + e, v4u{static_cast<uint32_t>(op[0]), static_cast<uint32_t>(op[1]),
                             static_cast<uint32_t>(op[2]), static_cast<uint32_t>(op[3])});
  }

  if (KONLY) return;
  if (job.kst) {
    // the tokens' signs as +/-1 bf16, transposed exactly as V^T below
    uint16_t* sout = job.kst + blk * static_cast<int64_t>(job.dpad) * kPackTok;
    for (int g = threadIdx.x; g < job.dpad * 8; g += kThreads) {
      const int c = g >> 3, q = g & 7;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t h2[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int key = vt_slot_key(8 * q + 2 * k + e);
          if (c < d && n0 + key < job.N) {
            const uint32_t neg = (sb[key * 4 * W + (c >> 3)] >> (c & 7)) & 1u;
            h2[e] = neg ? 0xBF80u : 0x3F80u;
          }
        }
        w[k] = h2[0] | (h2[1] << 16);
      }
      const int pos = q ^ ((c >> 1) & 7);
      *reinterpret_cast<uint4*>(sout + c * kPackTok + pos * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  if (job.vq) {
    kv_codes(job, blk, bh, tile, vs, stride, reinterpret_cast<float*>(vs + kPackTok * stride), sp);
    return;
  }
  if (!job.vt) return;

  // V^T
  uint16_t* out = job.vt + blk * static_cast<int64_t>(job.dpad) * kPackTok;
  for (int g = threadIdx.x; g < job.dpad * 8; g += kThreads) {
    const int c = g >> 3, q = g & 7;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t lo = 0, hi = 0;
      const int k0 = vt_slot_key(8 * q + 2 * k), k1 = vt_slot_key(8 * q + 2 * k + 1);
      if (c < d) {
        lo = vs[k0 * stride + c];
        hi = vs[k1 * stride + c];
      } else if (c == d || c == d + 4) {
        lo = (n0 + k0 < job.N) ? 0x3F80u : 0u;
        hi = (n0 + k1 < job.N) ? 0x3F80u : 0u;
      }
      w[k] = lo | (hi << 16);
    }
    const int pos = q ^ ((c >> 1) & 7);
    stream_out(out + c * kPackTok + pos * 8, v4u{w[0], w[1], w[2], w[3]});
  }
}

// 8-bit value codes of one tile ("Cuantizacion Hibrida": the values take a
// per-channel 8-bit quantization).  Channel c of head (b, h) has scale
// s_c = max_j |v_jc| / 127 over all N keys, the maximum of the tile maxima
// the previous launch wrote; the code of v is round-half-even(v * (127 /
// max)), the division correctly rounded.  The tile is written as dpad rows
// of 64 bytes in the order of the fused kernel's int8 operands: within each
// 32-key block, slot 16h + 4g + i holds key 8g + 4h + i (the order in which
// a lane of the QK result holds its keys), and the four 16-byte chunks
// q = 2 block + h of row c sit at chunk position q ^ ((c >> 2) & 3), so that
// the 16 rows one quarter-wave reads hit 16 different bank groups.  The
// codes of each channel are summed over the tile's keys into vcsum.
__device__ void kv_codes(const KvJob& job, int64_t blk, int64_t bh, int tile, const uint16_t* vs, int stride,
                         float* sinv, float* red) {
  const int tiles = job.Npad / kPackTok, n0 = tile * kPackTok;
  // The head's channel maxima from the tile maxima, with every thread: thread
  // (r, g) takes the maxima of channels 4g..4g+3 over tiles r, r + R, ...
  // (16-byte loads, all issued before they are used), then R partial maxima
  // per channel meet in `red` (the partial-sum scratch, free again here:
  // R * dpad <= 4 * kThreads floats).
  const int nc4 = job.dpad / 4, R = kThreads / nc4;
  const int g = threadIdx.x % nc4, r = threadIdx.x / nc4;
  __syncthreads();  // the key scales are done with `red`
  if (r < R) {
    const float4* vp = reinterpret_cast<const float4*>(job.vpart) + bh * tiles * nc4 + g;
    float4 m = make_float4(0.0f, 0.0f, 0.0f, 0.0f);  // maxima of |v| are >= 0
#pragma unroll 4
    for (int t = r; t < tiles; t += R) {
      const float4 x = vp[t * nc4];
      m = make_float4(fmaxf(m.x, x.x), fmaxf(m.y, x.y), fmaxf(m.z, x.z), fmaxf(m.w, x.w));
    }
    reinterpret_cast<float4*>(red)[r * nc4 + g] = m;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < job.dpad; c += kThreads) {
    float m = 0.0f;
    for (int i = 0; i < R; ++i) m = fmaxf(m, red[i * job.dpad + c]);
    sinv[c] = m > 0.0f ? __fdiv_rn(127.0f, m) : 0.0f;
    if (tile == 0) job.vscale[bh * job.dpad + c] = __fdiv_rn(m, 127.0f);
  }
  __syncthreads();
  int8_t* out = job.vq + blk * static_cast<int64_t>(job.dpad) * kPackTok;
  // (channel, chunk) pairs; the four chunks of a channel are in 4
  // consecutive lanes, and every wave that enters an iteration is full
  // (dpad * 4 is a multiple of 128)
  for (int e = threadIdx.x; e < job.dpad * 4; e += kThreads) {
    const int c = e >> 2, q = e & 3, b = q >> 1, h = q & 1;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    int sum = 0;
    if (c < job.d) {
      const float inv = sinv[c];
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) {
        const int key = 32 * b + 8 * (sl >> 2) + 4 * h + (sl & 3);
        int code = 0;
        if (n0 + key < job.N) code = static_cast<int>(rintf(bf16_to_f32(vs[key * stride + c]) * inv));
        sum += code;
        w[sl >> 2] |= (static_cast<uint32_t>(code) & 0xffu) << (8 * (sl & 3));
      }
    }
    const int pos = q ^ ((c >> 2) & 3);
    *reinterpret_cast<uint4*>(out + c * kPackTok + pos * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    if (q == 0 && sum != 0) atomicAdd(job.vcsum + bh * job.dpad + c, sum);
  }
}

// ---------------------------------------------------------------- vstat ---
// Channel maxima of |v| over one 64-token tile (tokens past N count as 0).
__device__ void vstat_block(const VstatJob& job, int64_t blk, unsigned char* smem) {
  const int d = job.d, C = d / 8;
  const int tiles = job.Npad / kPackTok;
  const int64_t bh = blk / tiles;
  const int tile = static_cast<int>(blk - bh * tiles), n0 = tile * kPackTok;
  unsigned* smax = reinterpret_cast<unsigned*>(smem);  // float bits; |v| >= 0 orders like the bits
  for (int c = threadIdx.x; c < job.dpad; c += kThreads) smax[c] = 0u;
  __syncthreads();
  const int rows = job.N - n0 < kPackTok ? job.N - n0 : kPackTok;
  const int64_t b = bh / job.H, hh = bh - b * job.H;
  const uint16_t* vbase = job.v + token_offset(job.vs, b, hh, n0);
  uint4 vr[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int g = threadIdx.x + i * kThreads;
    vr[i] = make_uint4(0u, 0u, 0u, 0u);
    if (g < rows * C) {
      const int tok = g / C, ch = g - tok * C;
      vr[i] = *reinterpret_cast<const uint4*>(vbase + tok * job.vs.sn + ch * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int g = threadIdx.x + i * kThreads;
    if (g < rows * C) {
      const int ch = g % C;
      const uint32_t wv[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        atomicMax(smax + 8 * ch + 2 * k, __float_as_uint(fabsf(bf16_to_f32(static_cast<uint16_t>(wv[k] & 0xffffu)))));
        atomicMax(smax + 8 * ch + 2 * k + 1, __float_as_uint(fabsf(bf16_to_f32(static_cast<uint16_t>(wv[k] >> 16)))));
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < job.dpad; c += kThreads) {
    job.vpart[blk * job.dpad + c] = __uint_as_float(smax[c]);
    if (tile == 0) job.vcsum[bh * job.dpad + c] = 0;
  }
}

// ---------------------------------------------------------------- bias ----
// One wave per row of the padded table, four rows per block:
// rows kBiasPadRows..kBiasPadRows + 2gh-2 hold the table rows dy = 0..2gh-2;
// the kBiasPadRows rows on each side are -inf (the fused kernel's windows
// reach them only for padded tokens).  Each row is 4 shifted copies of Lpad
// floats:
// R[u] = log2e * T[h, dy, 2gw-2-u] for 0 <= u <= 2gw-2 (else 0), and copy s
// holds C_s[v] = R[v+s].
__device__ void bias_block(const BiasJob& job, int64_t blk) {
  const int rows = 2 * job.gh - 1, cols = 2 * job.gw - 1;
  const int prow = rows + 2 * kBiasPadRows;
  const int lane = threadIdx.x & 63;
  // one wave per padded row; padded row `row` = h * prow + dyp
  const int64_t row = blk * kBiasRowsPerBlock + (threadIdx.x >> 6);
  if (row >= job.nrows) return;  // uniform in the wave; no barrier follows
  const int64_t h = row / prow;
  const int dyp = static_cast<int>(row - h * prow), dy = dyp - kBiasPadRows;
  const bool inside = dy >= 0 && dy < rows;
  // flipped: T'[dy][x] = T[rows-1-dy][cols-1-x]
  const uint16_t* trow = job.table + (h * rows + (inside ? (job.flip ? rows - 1 - dy : dy) : 0)) * cols;
  float4* out = reinterpret_cast<float4*>(job.bias4 + row * 4 * static_cast<int64_t>(job.Lpad));
  // Every table entry of the lane's 16-byte pieces is loaded before any
  // piece is stored, and every load is issued unconditionally (an entry the
  // piece does not take reads column 0 and is discarded): loads under a
  // condition would each wait for the one before.  Lpad % 4 == 0: the four
  // floats of a piece lie in one copy s.
  uint16_t raw[kBiasPieces][4];
  bool take[kBiasPieces][4];
#pragma unroll
  for (int i = 0; i < kBiasPieces; ++i) {
    const int e = 4 * (lane + 64 * i), s = e / job.Lpad, v = e - s * job.Lpad;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int u = v + t + s;
      take[i][t] = inside && e < 4 * job.Lpad && u <= cols - 1;
      const int uc = take[i][t] ? u : 0;
      raw[i][t] = trow[job.flip ? uc : cols - 1 - uc];
    }
  }
  float val[kBiasPieces][4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kBiasPieces; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // Padding rows are -inf: the only (query, key) pairs that reach them
      // involve a padded token.  They keep the fused kernel's window reads
      // inside the rows; that kernel masks padded keys itself, since a
      // padded key seen from a query on grid row >= 1 falls on a real row.
      val[i][t] = take[i][t] ? kLog2e * bf16_to_f32(raw[i][t]) : (inside ? 0.0f : -INFINITY);
      if (inside) m = fmaxf(m, fabsf(val[i][t]));
    }
#pragma unroll
  for (int i = 0; i < kBiasPieces; ++i)
    if (lane + 64 * i < job.Lpad)
      stream_out(out + lane + 64 * i, v4u{__float_as_uint(val[i][0]), __float_as_uint(val[i][1]),
                                          __float_as_uint(val[i][2]), __float_as_uint(val[i][3])});
  // row maximum of |entry| * log2e, for the logit bound
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0 && inside) job.row_max[h * rows + dy] = m;
}

// ------------------------------------------------------------- expansion --
// Row (h, i) of the dense bias (see ExpandJob): 8 consecutive keys per
// thread and 16-byte stores.  Keys on one grid row read consecutive table
// columns in reverse order (xi - xj falls as xj rises).
__device__ void expand_row(const ExpandJob& j, int64_t blk) {
  const int h = static_cast<int>(blk / j.Npad), i = static_cast<int>(blk - static_cast<int64_t>(h) * j.Npad);
  const int rows = 2 * j.gh - 1, cols = 2 * j.gw - 1;
  const uint16_t* tab = j.table + static_cast<int64_t>(h) * rows * cols;
  uint16_t* out = j.out + (static_cast<int64_t>(h) * j.Npad + i) * j.Npad;
  const int yi = i / j.gw, xi = i - yi * j.gw;
  for (int j0 = 8 * threadIdx.x; j0 < j.Npad; j0 += 8 * kThreads) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (i < j.N) {
      int yj = j0 / j.gw, xj = j0 - yj * j.gw;
      // the eight loads go out unconditionally (a key past N reads the
      // table's centre entry and is dropped), so that none waits for another
      uint32_t val[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool real = j0 + e < j.N;
        val[e] = tab[real ? (yi - yj + j.gh - 1) * cols + (xi - xj + j.gw - 1) : (j.gh - 1) * cols + j.gw - 1];
        val[e] = real ? val[e] : 0u;
        if (++xj == j.gw) {
          xj = 0;
          ++yj;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e >> 1] |= val[e] << (16 * (e & 1));
    }
    stream_out(out + j0, v4u{w[0], w[1], w[2], w[3]});
  }
}

// FWD: the forward's jobs alone (keys without values, bias rows, the
// expanded bias), compiled without the others so that the kernel needs
// fewer registers (63 instead of 95 VGPRs, no scratch) and more of its
// blocks are resident at once.
template <bool FWD>
__global__ void __launch_bounds__(kThreads) prologue_kernel(PrologueArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int64_t blk = blockIdx.x;
  if (!FWD) {
    if (blk < a.pack_blocks) {
      pack_block(a.pack, blk, smem);
      return;
    }
    blk -= a.pack_blocks;
  }
  if (blk < a.kv_blocks) {
    kv_block<FWD>(a.kv, blk, smem);
    return;
  }
  blk -= a.kv_blocks;
  if (blk < a.bias_blocks) {
    bias_block(a.bias, blk);
    return;
  }
  blk -= a.bias_blocks;
  if (FWD) {
    if (blk < a.expand_blocks) expand_row(a.expand, blk);
    return;
  }
  if (blk < a.vstat_blocks) {
    vstat_block(a.vstat, blk, smem);
    return;
  }
  blk -= a.vstat_blocks;
  if (blk < a.bias2_blocks) {
    bias_block(a.bias2, blk);
    return;
  }
  blk -= a.bias2_blocks;
  if (blk < a.dtr_blocks) {
    // 32 table entries per block, each summed by 8 threads over consecutive
    // runs of its B * nqt shares (i = b nqt + qt); the 8 partial sums meet in
    // LDS and are added in a fixed order, so the result is the same on every
    // run.
    const DtReduceJob& j = a.dtr;
    const int w2 = 2 * j.gw - 1, rows = 2 * j.gh - 1;
    const int64_t total = static_cast<int64_t>(j.H) * rows * w2;
    const int64_t e = blk * kDtEntries + (threadIdx.x % kDtEntries);
    const int grp = threadIdx.x / kDtEntries;
    const int n = j.B * j.nqt, per = (n + kDtGroups - 1) / kDtGroups;
    float acc = 0.0f;
    if (e < total) {
      const int h = static_cast<int>(e / (rows * w2));
      const int rem = static_cast<int>(e - static_cast<int64_t>(h) * rows * w2);
      const int dyi = rem / w2, col = rem - dyi * w2;
      // the query tile's first table row by a multiplication when gw
      // divides 128
      const int step = (j.rows_mode && 128 % j.gw == 0) ? 128 / j.gw : -1;
      const int i0 = grp * per, i1 = (i0 + per < n) ? i0 + per : n;
      int b = i0 / j.nqt, qt = i0 - b * j.nqt;
      // eight loads in flight at a time: a share that does not cover the
      // entry (or lies past the run) reads the first element instead and
      // adds zero
      for (int i = i0; i < i1; i += 8) {
        float v[8];
        bool use[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row0 = !j.rows_mode ? 0 : (step > 0 ? qt * step : (128 * qt) / j.gw);
          const int r = dyi - row0;
          use[u] = i + u < i1 && r >= 0 && r < j.prow;
          const int64_t off =
              ((static_cast<int64_t>(b) * j.H + h) * j.nqt + qt) * j.prow * w2 + r * w2 + col;
          v[u] = j.part[use[u] ? off : 0];
          if (++qt == j.nqt) {
            qt = 0;
            ++b;
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (use[u]) acc += v[u];
      }
    }
    __shared__ float dpart[kDtGroups][kDtEntries];
    dpart[grp][threadIdx.x % kDtEntries] = acc;
    __syncthreads();
    if (grp == 0 && e < total) {
      float sum = dpart[0][threadIdx.x];
      for (int g = 1; g < kDtGroups; ++g) sum += dpart[g][threadIdx.x];
      j.dtable[e] = sum;
    }
    return;
  }
  blk -= a.dtr_blocks;
  if (blk < a.lse_blocks) {
    const LseJob& j = a.lsej;
    const int64_t e = blk * kThreads + threadIdx.x;
    if (e < j.BH * j.Npad) {
      const int64_t bh = e / j.Npad;
      const int i = static_cast<int>(e - bh * j.Npad);
      j.out[e] = i < j.N ? j.in[bh * j.N + i] * kLog2e : 0.0f;
    }
    return;
  }
  blk -= a.lse_blocks;
  if (blk < a.delta_blocks) {
    // thread pair (2r, 2r + 1): row r of the launch, channel halves 0 and 1;
    // every lane reaches the exchange (rows past BH * Npad contribute 0)
    const DeltaJob& j = a.delta;
    const int64_t e = blk * kThreads + threadIdx.x, row = e >> 1;
    const int half = static_cast<int>(e & 1);
    const bool inrow = row < j.BH * j.Npad;
    const int64_t bh = inrow ? row / j.Npad : 0;
    const int i = inrow ? static_cast<int>(row - bh * j.Npad) : 0;
    const bool valid = inrow && i < j.N;
    float part = 0.0f;
    if (valid) {
      const uint16_t* orow = j.o + (bh * j.N + i) * j.d;
      const uint16_t* grow = j.dout + (bh * j.N + i) * j.d;
      for (int t = 0; t < j.d / 16; ++t) {
        const uint4 ro = *reinterpret_cast<const uint4*>(orow + 16 * t + 8 * half);
        const uint4 rg = *reinterpret_cast<const uint4*>(grow + 16 * t + 8 * half);
        const uint32_t wo[4] = {ro.x, ro.y, ro.z, ro.w}, wg[4] = {rg.x, rg.y, rg.z, rg.w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          part += bf16_to_f32(static_cast<uint16_t>(wo[k] & 0xffffu)) * bf16_to_f32(static_cast<uint16_t>(wg[k] & 0xffffu)) +
                  bf16_to_f32(static_cast<uint16_t>(wo[k] >> 16)) * bf16_to_f32(static_cast<uint16_t>(wg[k] >> 16));
      }
    }
    const float sum = part + __shfl_xor(part, 1, 64);
    if (inrow && half == 0) j.delta[row] = valid ? sum : 0.0f;
    return;
  }
  blk -= a.delta_blocks;
  if (blk < a.expand_blocks) expand_row(a.expand, blk);
}

int launch_prologue(const PrologueArgs& a, void* stream) {
  const int64_t blocks = a.pack_blocks + a.kv_blocks + a.bias_blocks + a.vstat_blocks + a.bias2_blocks +
                        a.dtr_blocks + a.lse_blocks + a.delta_blocks + a.expand_blocks;
  const KvJob& kv = a.kv;
  const bool keys_only = a.kv_blocks == 0 || (!kv.vt && !kv.vq && !kv.vmax && !kv.vnat && !kv.kst);
  const bool fwd = keys_only && a.pack_blocks == 0 && a.vstat_blocks == 0 && a.bias2_blocks == 0 &&
                   a.dtr_blocks == 0 && a.lse_blocks == 0 && a.delta_blocks == 0;
  if (fwd) {
    // the keys-only tile needs the partial sums and sign words alone
    const int lds = a.kv_blocks > 0 ? prologue_lds(kv.d, false) : 0;
    hipLaunchKernelGGL(prologue_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), lds,
                       static_cast<hipStream_t>(stream), a);
  } else {
    hipLaunchKernelGGL(prologue_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), a.lds,
                       static_cast<hipStream_t>(stream), a);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace ba
