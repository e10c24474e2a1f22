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
//         O^T accumulator keeps one query per lane, so the softmax
//         rescale and the final 1/l are per-lane scalars.
//
// Workgroup: 4 waves x 32 queries = 128 queries of one (b, h).  Each 64-key
// step stages the fp4 key operands (expanded once from the packed bits), the
// key scales, the V^T tile and a window of the bias table in LDS.  Softmax is
// the exact online form in base 2: running row max m, l and O rescaled by
// 2^(m_old - m_new), with the rescale skipped while the max grows by at most
// 8 (P values stay <= 2^8, so nothing overflows).
#include "ba_internal.h"

namespace ba {

template <int NCH, int CB, int BIAS>
__global__ void __launch_bounds__(kThreads) attn_fwd_kernel(FwdArgs a) {
  constexpr int DPAD = 32 * CB;
  __shared__ __attribute__((aligned(16))) v4i s_k[NCH * kBN * 2];
  __shared__ __attribute__((aligned(16))) float s_ak[kBN];
  __shared__ __attribute__((aligned(16))) int s_gk[kBN];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[DPAD * kVtStride];
  extern __shared__ __attribute__((aligned(16))) float s_bias[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;

  int wg = blockIdx.x;
  if (a.xcd_remap) {
    const int per = a.nwg >> 3;
    wg = (wg & 7) * per + (wg >> 3);
  }
  const int bh = wg / a.nqt, qt = wg - bh * a.nqt;
  const int head = bh % a.H;
  const int q0 = qt * kBM;
  const int qi = q0 + wave * 32 + li;
  const int64_t tokbase = static_cast<int64_t>(bh) * a.Npad;

  // Query operands: word 2c + lh of this lane's query, as fp4 +/-1.
  v4i qop[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int word = 2 * c + lh;
    const uint32_t w = word < a.W ? a.qbits[(tokbase + qi) * a.W + word] : 0u;
    qop[c] = expand_signs_fp4(w, fp4_magnitude(word_valid(a.d, word)));
  }
  const float aq = a.alpha_q[tokbase + qi] * a.qscale;

  int yq = 0, xq = 0, fidx = 0, bsel = 0, yq_lo = 0;
  if (BIAS != kBiasNone) {
    yq = qi / a.gw;
    xq = qi - yq * a.gw;
  }
  if (BIAS == kBiasRows) {
    bsel = (a.gw - 1 - xq) & 3;
    yq_lo = q0 / a.gw;
  }
  if (BIAS == kBiasTable) {
    const int yc = yq < a.gh ? yq : a.gh - 1;
    fidx = (yc + a.gh - 1) * (2 * a.gw - 1) + xq + a.gw - 1;
    const int n = (2 * a.gh - 1) * (2 * a.gw - 1);
    const uint16_t* t = a.table + static_cast<int64_t>(head) * n;
    for (int e = tid; e < n; e += kThreads) s_bias[e] = kLog2e * bf16_to_f32(t[e]);
  }

  v16f oacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) oacc[cb] = v16f{};
  float lsum = 0.0f;
  float mrow = -INFINITY;

  const int nkt = (a.N + kBN - 1) / kBN;
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBN;
    __syncthreads();
    // ---- stage the key tile -------------------------------------------
    for (int e = tid; e < NCH * kBN * 2; e += kThreads) {
      const int c = e / (kBN * 2), key = (e >> 1) & (kBN - 1), word = 2 * c + (e & 1);
      const uint32_t w = word < a.W ? a.kbits[(tokbase + k0 + key) * a.W + word] : 0u;
      s_k[e] = expand_signs_fp4(w, fp4_magnitude(word_valid(a.d, word)));
    }
    if (tid < kBN) {
      s_ak[tid] = a.alpha_k[tokbase + k0 + tid];
      if (BIAS == kBiasTable) {
        const int j = (k0 + tid < a.N) ? k0 + tid : a.N - 1;
        const int yj = j / a.gw;
        s_gk[tid] = yj * (2 * a.gw - 1) + (j - yj * a.gw);
      }
    }
    for (int e = tid; e < DPAD * 8; e += kThreads) {
      const int c = e >> 3, q = e & 7;
      *reinterpret_cast<uint4*>(s_vt + c * kVtStride + 8 * q) = *reinterpret_cast<const uint4*>(
          a.vt + (static_cast<int64_t>(bh) * DPAD + c) * a.Npad + k0 + 8 * q);
    }
    int dy_min = 0;
    if (BIAS == kBiasRows) {
      dy_min = yq_lo - (k0 + kBN - 1) / a.gw;
      const int per = 4 * a.Lpad;
      const int nvec = a.win_rows * a.Lpad;  // float4 count
      const int rows_tab = 2 * a.gh - 1;
      for (int e = tid; e < nvec; e += kThreads) {
        const int r = (4 * e) / per;
        const int dyidx = dy_min + r + a.gh - 1;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (dyidx >= 0 && dyidx < rows_tab)
          val = *reinterpret_cast<const float4*>(
              a.bias4 + (static_cast<int64_t>(head) * rows_tab + dyidx) * per + (4 * e - r * per));
        *reinterpret_cast<float4*>(s_bias + 4 * e) = val;
      }
    }
    __syncthreads();

    // ---- QK: D for 64 keys x 32 queries (two 32x32 blocks) -------------
    v16f sblk[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      sblk[blk] = v16f{};
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        sblk[blk] = mfma_signs_32x32x64(s_k[(c * kBN + blk * 32 + li) * 2 + lh], qop[c], sblk[blk]);
    }

    // ---- scores in base 2: D * alpha_k * (alpha_q scale log2e) + log2e b --
    float sc[2][16];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      int brow = 0, bu0 = 0;
      if (BIAS == kBiasRows) {
        const int kb0 = k0 + blk * 32;
        const int yk = kb0 / a.gw, xk0 = kb0 - yk * a.gw;
        brow = yq - yk - dy_min;
        bu0 = a.gw - 1 - xq + xk0 + 4 * lh - bsel;
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float4 ak = *reinterpret_cast<const float4*>(s_ak + blk * 32 + 8 * b + 4 * lh);
        float4 bias = make_float4(0.f, 0.f, 0.f, 0.f);
        if (BIAS == kBiasRows) {
          bias = *reinterpret_cast<const float4*>(s_bias + (brow * 4 + bsel) * a.Lpad + bu0 + 8 * b);
        } else if (BIAS == kBiasTable) {
          const int4 g = *reinterpret_cast<const int4*>(s_gk + blk * 32 + 8 * b + 4 * lh);
          bias = make_float4(s_bias[fidx - g.x], s_bias[fidx - g.y], s_bias[fidx - g.z], s_bias[fidx - g.w]);
        }
        sc[blk][4 * b + 0] = fmaf(sblk[blk][4 * b + 0] * ak.x, aq, bias.x);
        sc[blk][4 * b + 1] = fmaf(sblk[blk][4 * b + 1] * ak.y, aq, bias.y);
        sc[blk][4 * b + 2] = fmaf(sblk[blk][4 * b + 2] * ak.z, aq, bias.z);
        sc[blk][4 * b + 3] = fmaf(sblk[blk][4 * b + 3] * ak.w, aq, bias.w);
      }
    }
    if (k0 + kBN > a.N) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + blk * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (key >= a.N) sc[blk][r] = -INFINITY;
        }
    }

    // ---- online softmax (exact, base 2, lazy rescale) -------------------
    float mt = sc[0][0];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[blk][r]);
    mt = max_halves(mt);
    const float mnew = fmaxf(mrow, mt);
    if (__any(mnew > mrow + 8.0f)) {
      const float f = fast_exp2(mrow - mnew);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) oacc[cb] *= f;
      lsum *= f;
      mrow = mnew;
    }
    uint32_t pk[2][8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pk[blk][j] = pack_bf16x2(fast_exp2(sc[blk][2 * j] - mrow), fast_exp2(sc[blk][2 * j + 1] - mrow));
        lsum = add_bf16x2(pk[blk][j], lsum);
      }

    // ---- P.V: O^T[c][i] += sum_k V^T[c][k] P^T[k][i] -------------------
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int blk = p >> 1, off = (p & 1) * 4;
      const v4u pw = {pk[blk][off], pk[blk][off + 1], pk[blk][off + 2], pk[blk][off + 3]};
      const v8bf pop = __builtin_bit_cast(v8bf, pw);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const v8bf vop = *reinterpret_cast<const v8bf*>(s_vt + (cb * 32 + li) * kVtStride + 16 * p + 8 * lh);
        oacc[cb] = mfma_bf16_32x32x16(vop, pop, oacc[cb]);
      }
    }
  }

  // ---- epilogue: O = O^T / l, bf16, one query per lane --------------------
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) pin_uniform(oacc[cb]);
  const float inv = 1.0f / sum_halves(lsum);
  if (qi < a.N) {
    uint16_t* orow = a.o + (static_cast<int64_t>(bh) * a.N + qi) * a.d;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int c0 = cb * 32 + 8 * b + 4 * lh;
        if (c0 < a.d) {
          uint2 w;
          w.x = pack_bf16x2(oacc[cb][4 * b + 0] * inv, oacc[cb][4 * b + 1] * inv);
          w.y = pack_bf16x2(oacc[cb][4 * b + 2] * inv, oacc[cb][4 * b + 3] * inv);
          *reinterpret_cast<uint2*>(orow + c0) = w;
        }
      }
  }
}

int fwd_dynamic_lds(const FwdArgs& a, int mode) {
  if (mode == kBiasRows) return a.win_rows * 4 * a.Lpad * 4;
  if (mode == kBiasTable) return (2 * a.gh - 1) * (2 * a.gw - 1) * 4;
  return 0;
}

template <int NCH, int CB>
static int launch_nc(const FwdArgs& a, int mode, void* stream) {
  const int lds = fwd_dynamic_lds(a, mode);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(a.nwg), block(kThreads);
  switch (mode) {
    case kBiasNone:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, kBiasNone>), grid, block, lds, s, a);
      break;
    case kBiasRows:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, kBiasRows>), grid, block, lds, s, a);
      break;
    default:
      hipLaunchKernelGGL((attn_fwd_kernel<NCH, CB, kBiasTable>), grid, block, lds, s, a);
      break;
  }
  return static_cast<int>(hipGetLastError());
}

int launch_attention(const FwdArgs& a, int mode, void* stream) {
  const int cb = a.dpad / 32;
  switch (cb) {
    case 1: return launch_nc<1, 1>(a, mode, stream);
    case 2: return launch_nc<1, 2>(a, mode, stream);
    case 3: return launch_nc<2, 3>(a, mode, stream);
    case 4: return launch_nc<2, 4>(a, mode, stream);
    case 5: return launch_nc<3, 5>(a, mode, stream);
    case 6: return launch_nc<3, 6>(a, mode, stream);
    case 7: return launch_nc<4, 7>(a, mode, stream);
    case 8: return launch_nc<4, 8>(a, mode, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace ba
