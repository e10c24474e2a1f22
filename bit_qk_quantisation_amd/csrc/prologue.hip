// Prologue kernel of the BinaryAttention forward, plus the standalone sign
// pack.
//
// One launch does three independent jobs, split by block index:
//   * pack: per token, the scale alpha = mean |x| over d and the packed sign
//     words (s_i = mu sign(q_i), "Representaciones Binarias Escaladas" of
//     the BinaryAttention summary).  It covers Q and K, or a single tensor
//     for ba_pack_signs.  For K the signs are written as the fp4 +/-1 MFMA
//     operand tiles the fused kernel copies straight into LDS.
//   * vt: a key-major copy of V (V^T, bf16 [BH][dpad][Npad]) whose keys are
//     permuted inside each group of 16 to match the P.V operand order of the
//     fused kernel.
//   * bias rows: the relative-position table ("Mejora mediante Sesgo") as
//     float32 * log2(e), with the dx axis reversed, in four copies shifted
//     by 0..3 entries, so that any 4 consecutive entries can be read with
//     one aligned 16-byte LDS load.
// All three are bound by HBM traffic.  Loads are 16-byte and coalesced.
#include "ba_internal.h"

namespace ba {

// ---------------------------------------------------------------- pack ----
// One block = 64 tokens.  Each thread takes 8-channel chunks (16 bytes), so
// consecutive threads read consecutive 16-byte pieces of the rows.  Sign
// bytes and partial |x| sums meet in LDS, then words and scales are written.
constexpr int kPackTok = 64;

__device__ void pack_block(const PackJob& job, int64_t blk, unsigned char* smem) {
  const int d = job.d, W = job.W, C = d / 8;
  const int64_t T = job.BH * static_cast<int64_t>(job.Npad);
  const int64_t t0 = blk * kPackTok;
  uint32_t* sw = reinterpret_cast<uint32_t*>(smem);            // [64][W] words
  float* sp = reinterpret_cast<float*>(smem + kPackTok * 8 * 4);  // [64][33]

  for (int e = threadIdx.x; e < kPackTok * W; e += blockDim.x) sw[e] = 0u;
  __syncthreads();

  unsigned char* sb = reinterpret_cast<unsigned char*>(sw);
  for (int g = threadIdx.x; g < kPackTok * C; g += blockDim.x) {
    const int tok = g / C, ch = g - tok * C;
    const int64_t t = t0 + tok;
    uint32_t byte = 0;
    float part = 0.0f;
    if (t < T) {
      const int64_t bh = t / job.Npad;
      const int n = static_cast<int>(t - bh * job.Npad);
      if (n < job.N) {
        const uint4 raw = *reinterpret_cast<const uint4*>(
            job.x + ((bh * job.N + n) * d + ch * 8));
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
        float a[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float lo = bf16_to_f32(static_cast<uint16_t>(wv[k] & 0xffffu));
          const float hi = bf16_to_f32(static_cast<uint16_t>(wv[k] >> 16));
          byte |= neg_bit(lo) << (2 * k);
          byte |= neg_bit(hi) << (2 * k + 1);
          a[2 * k] = fabsf(lo);
          a[2 * k + 1] = fabsf(hi);
        }
        part = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
      }
    }
    // channel 8*ch + b -> word ch/4, bit 8*(ch%4) + b: byte ch of the
    // token's little-endian word array.
    sb[tok * 4 * W + ch] = static_cast<unsigned char>(byte);
    sp[tok * 33 + ch] = part;
  }
  __syncthreads();

  if (job.bits != nullptr) {
    for (int e = threadIdx.x; e < kPackTok * W; e += blockDim.x) {
      const int tok = e / W;
      const int64_t t = t0 + tok;
      if (t < T) job.bits[t * W + (e - tok * W)] = sw[e];
    }
  }
  if (job.kop != nullptr) {
    // fp4 +/-1 operands of the 64 keys (one key tile: blocks never straddle
    // tiles, Npad % 64 == 0), in the fused kernel's LDS order
    // [chunk][key][half][4 dwords]: word 2*chunk + half of the key, expanded
    // exactly as the fused kernel expands its query words.  Consecutive
    // threads write consecutive 16-byte pieces.
    uint4* dst = reinterpret_cast<uint4*>(job.kop) + blk * (kPackTok * 2 * job.nch);
    for (int e = threadIdx.x; e < kPackTok * 2 * job.nch; e += blockDim.x) {
      const int ch = e >> 7, key = (e >> 1) & (kPackTok - 1), w = 2 * ch + (e & 1);
      const uint32_t word = w < W ? sw[key * W + w] : 0u;
      const v4i op = expand_signs_fp4(word, fp4_magnitude(word_valid(d, w)));
      dst[e] = make_uint4(static_cast<uint32_t>(op[0]), static_cast<uint32_t>(op[1]),
                          static_cast<uint32_t>(op[2]), static_cast<uint32_t>(op[3]));
    }
  }
  if (threadIdx.x < kPackTok) {
    const int tok = threadIdx.x;
    const int64_t t = t0 + tok;
    if (t < T) {
      float* v = sp + tok * 33;
      // pairwise sum in a fixed order: error <= ceil(log2 d) ulps-ish
      for (int s = 1; s < C; s *= 2)
        for (int i = 0; i + s < C; i += 2 * s) v[i] += v[i + s];
      const int64_t bh = t / job.Npad;
      const int n = static_cast<int>(t - bh * job.Npad);
      job.alpha[t] = (n < job.N) ? v[0] / static_cast<float>(d) : 0.0f;
    }
  }
  if (job.alpha_max != nullptr && threadIdx.x < 64) {
    // Block maximum of alpha (64 tokens, never straddling heads since Npad is
    // a multiple of 64).  alpha >= 0, so the lane fold starts from 0.
    const int tok = threadIdx.x;
    const int64_t t = t0 + tok;
    float m = 0.0f;
    if (t < T) {
      const int64_t bh = t / job.Npad;
      const int n = static_cast<int>(t - bh * job.Npad);
      if (n < job.N) m = sp[tok * 33] / static_cast<float>(d);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (tok == 0) job.alpha_max[blk] = m;
  }
}

// ------------------------------------------------------------------ vt ----
// One block = one (b,h) and 64 keys.  Loads the 64 x d tile row-major into
// LDS, then writes the tile's dpad rows of 64 keys (zeros past N and past d,
// except rows d and d+4 when d is not a multiple of 32: those hold 1.0 for
// every key < N) as one contiguous dpad x 128-byte block, in the order the fused kernel
// copies straight into LDS:
//   * keys are permuted inside each group of 16 into the P.V slot order
//     (slots 8h..8h+3 = keys 4h..4h+3, slots 8h+4..8h+7 = keys 8+4h..8+4h+3);
//   * the eight 16-byte chunks of row c are stored at chunk position
//     q ^ ((c >> 1) & 7), so that 16 lanes reading one chunk from 16
//     consecutive rows touch 16 different 4-bank groups.
__device__ __forceinline__ int vt_slot_key(int slot) {
  const int g = slot >> 4, s16 = slot & 15, hh = s16 >> 3, s = s16 & 7;
  return g * 16 + (s < 4 ? 4 * hh + s : 8 + 4 * hh + (s - 4));
}

__device__ void vt_block(const VtJob& job, int64_t blk, unsigned char* smem) {
  const int d = job.d, C = d / 8, stride = d + 8;  // bf16 units
  const int tiles = job.Npad / 64;
  const int64_t bh = blk / tiles;
  const int tile = static_cast<int>(blk - bh * tiles), n0 = tile * 64;
  uint16_t* t = reinterpret_cast<uint16_t*>(smem);  // [64][d+8]

  for (int g = threadIdx.x; g < 64 * C; g += blockDim.x) {
    const int key = g / C, ch = g - key * C;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (n0 + key < job.N)
      raw = *reinterpret_cast<const uint4*>(job.v + ((bh * job.N + n0 + key) * d + ch * 8));
    *reinterpret_cast<uint4*>(t + key * stride + ch * 8) = raw;
  }
  __syncthreads();
  uint16_t* out = job.vt + (bh * tiles + tile) * static_cast<int64_t>(job.dpad) * 64;
  for (int g = threadIdx.x; g < job.dpad * 8; g += blockDim.x) {
    const int c = g >> 3, q = g & 7;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t lo = 0, hi = 0;
      if (c < d) {
        lo = t[vt_slot_key(8 * q + 2 * k) * stride + c];
        hi = t[vt_slot_key(8 * q + 2 * k + 1) * stride + c];
      } else if (c == d || c == d + 4) {
        // rows of ones: the P.V product then also yields the row sums of P
        lo = (n0 + vt_slot_key(8 * q + 2 * k) < job.N) ? 0x3F80u : 0u;
        hi = (n0 + vt_slot_key(8 * q + 2 * k + 1) < job.N) ? 0x3F80u : 0u;
      }
      w[k] = lo | (hi << 16);
    }
    const int pos = q ^ ((c >> 1) & 7);
    *reinterpret_cast<uint4*>(out + c * 64 + pos * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------- bias ----
// One block = one row of the padded table: rows kBiasPadRows..kBiasPadRows +
// 2gh-2 hold the table rows dy = 0..2gh-2; the kBiasPadRows rows on each side
// are -inf (the fused kernel's windows reach them only for padded tokens).  Each row is 4 shifted copies of Lpad floats:
// R[u] = log2e * T[h, dy, 2gw-2-u] for 0 <= u <= 2gw-2 (else 0), and copy s
// holds C_s[v] = R[v+s].
__device__ void bias_block(const BiasJob& job, int64_t blk) {
  const int rows = 2 * job.gh - 1, cols = 2 * job.gw - 1;
  const int prow = rows + 2 * kBiasPadRows;
  const int64_t h = blk / prow;
  const int dyp = static_cast<int>(blk - h * prow), dy = dyp - kBiasPadRows;
  const bool inside = dy >= 0 && dy < rows;
  const uint16_t* trow = job.table + (h * rows + (inside ? dy : 0)) * cols;
  float* out = job.bias4 + (h * prow + dyp) * 4 * static_cast<int64_t>(job.Lpad);
  float m = 0.0f;
  for (int e = threadIdx.x; e < 4 * job.Lpad; e += blockDim.x) {
    const int s = e / job.Lpad, v = e - s * job.Lpad;
    const int u = v + s;
    // Padding rows are -inf: the only (query, key) pairs that reach them
    // involve a padded token, and a padded key must get probability 0.
    float val = inside ? 0.0f : -INFINITY;
    if (inside && u <= cols - 1) val = kLog2e * bf16_to_f32(trow[cols - 1 - u]);
    out[e] = val;
    if (inside) m = fmaxf(m, fabsf(val));
  }
  // row maximum of |entry| * log2e, for the logit bound
  __shared__ float wmax[kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0 && inside) {
    float r = wmax[0];
    for (int i = 1; i < static_cast<int>(blockDim.x >> 6); ++i) r = fmaxf(r, wmax[i]);
    job.row_max[h * rows + dy] = r;
  }
}

__global__ void __launch_bounds__(256) prologue_kernel(PrologueArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPrologueSmem];
  int64_t blk = blockIdx.x;
  for (int t = 0; t < a.npack; ++t) {
    if (blk < a.pack_blocks) {
      pack_block(a.pack[t], blk, smem);
      return;
    }
    blk -= a.pack_blocks;
  }
  if (blk < a.vt_blocks) {
    vt_block(a.vt, blk, smem);
    return;
  }
  blk -= a.vt_blocks;
  if (blk < a.bias_blocks) bias_block(a.bias, blk);
}

int launch_prologue(const PrologueArgs& a, void* stream) {
  const int64_t blocks = a.npack * a.pack_blocks + a.vt_blocks + a.bias_blocks;
  hipLaunchKernelGGL(prologue_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace ba
