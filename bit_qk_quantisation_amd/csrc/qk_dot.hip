// QK integer dots D_ij = <sign q_i, sign k_j> for every pair: the check hook
// for the similarity step of the BinaryAttention kernel ("XNOR y popcount",
// "Representaciones Binarias Escaladas").
//
// Route BA_ROUTE_MFMA_FP4 runs exactly the device code of the fused kernel
// (expand_signs_fp4 + mfma_signs_32x32x64).  Route BA_ROUTE_MFMA_INT8 takes
// the signs as +/-1 int8 on v_mfma_i32_32x32x32_i8 (32 channels a product,
// exact int32 sums).  Route BA_ROUTE_VALU_POPCOUNT takes d - 2 popcount(q XOR
// k) on the packed words with v_xor/v_bcnt.
//
// The row-sum form (route | BA_QK_ROWSUM) returns sum_j D_ij per query
// instead of the N x N matrix, so that it reads little and writes little: it
// times each route's QK arithmetic in the setting the fused kernel has (keys
// expanded once per 64-key tile into LDS and shared by a workgroup's 128
// queries, the queries' operands held in registers).
#include "ba_internal.h"

namespace ba {

// One wave = 32 queries x 32 keys; blockIdx.x covers 4 key blocks.
template <int NCH>
__global__ void __launch_bounds__(kThreads) qk_dot_mfma_kernel(DotArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int kb = blockIdx.x * 4 + wave;
  const int qb = blockIdx.y;
  const int64_t bh = blockIdx.z;
  if (kb * 32 >= a.N) return;  // whole wave leaves together; no barriers below
  const int qi = qb * 32 + li;
  const int kr = kb * 32 + li;
  const int64_t base = bh * a.N;
  v16f s = v16f{};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int word = 2 * c + lh;
    const uint32_t mag = fp4_magnitude(word_valid(a.d, word));
    const uint32_t wq = (qi < a.N && word < a.W) ? a.qbits[(base + qi) * a.W + word] : 0u;
    const uint32_t wk = (kr < a.N && word < a.W) ? a.kbits[(base + kr) * a.W + word] : 0u;
    s = mfma_signs_32x32x64(expand_signs_fp4(wk, mag), expand_signs_fp4(wq, mag), s);
  }
  pin_uniform(s);
  if (qi >= a.N) return;
  int32_t* row = a.dots + (base + qi) * a.N;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
    if (key < a.N) row[key] = static_cast<int32_t>(s[r]);
  }
}

// +/-1 int8 operand of 16 channels: bit c of `bits` (sign) -> byte c of the
// result, 0xff (-1) when set, 0x01 (+1) when clear, 0 where c >= nvalid.
__device__ __forceinline__ v4i expand_signs_i8(uint32_t bits, int nvalid) {
  v4i r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t nib = (bits >> (4 * k)) & 0xfu;
    // spread the four bits to bytes 0..3 (bit t -> bit 8 t)
    const uint32_t t = (nib | (nib << 7) | (nib << 14) | (nib << 21)) & 0x01010101u;
    const uint32_t bytes = 0x01010101u ^ (t * 0xfeu);
    const int keep = nvalid - 4 * k;  // channels of this group that exist
    const uint32_t mask = keep >= 4 ? 0xffffffffu : (keep <= 0 ? 0u : (1u << (8 * keep)) - 1u);
    r[k] = static_cast<int>(bytes & mask);
  }
  return r;
}

// Valid channels among the 16 of half `h` of 32-channel word `w`.
__device__ __forceinline__ int half_valid(int d, int w, int h) {
  const int v = d - 32 * w - 16 * h;
  return v < 0 ? 0 : (v > 16 ? 16 : v);
}

// One wave = 32 queries x 32 keys on +/-1 int8, 32 channels a product.
template <int W>
__global__ void __launch_bounds__(kThreads) qk_dot_i8_kernel(DotArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int kb = blockIdx.x * 4 + wave;
  const int qb = blockIdx.y;
  const int64_t bh = blockIdx.z;
  if (kb * 32 >= a.N) return;  // whole wave leaves together; no barriers below
  const int qi = qb * 32 + li;
  const int kr = kb * 32 + li;
  const int64_t base = bh * a.N;
  v16i s = v16i{};
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int nv = half_valid(a.d, w, lh);
    const uint32_t wq = (qi < a.N && w < a.W) ? a.qbits[(base + qi) * a.W + w] : 0u;
    const uint32_t wk = (kr < a.N && w < a.W) ? a.kbits[(base + kr) * a.W + w] : 0u;
    s = __builtin_amdgcn_mfma_i32_32x32x32_i8(expand_signs_i8(wk >> (16 * lh), nv),
                                              expand_signs_i8(wq >> (16 * lh), nv), s, 0, 0, 0);
  }
  if (qi >= a.N) return;
  int32_t* row = a.dots + (base + qi) * a.N;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
    if (key < a.N) row[key] = s[r];
  }
}

// ---- row sums: each route's QK arithmetic with little memory traffic -------
// Workgroup = 4 waves x 32 queries; key tiles of 64 are expanded once into
// LDS (the route's operand layout, zero for keys past N) and read by every
// wave, as the fused kernel reads its key tiles.
template <int ROUTE, int W>
__global__ void __launch_bounds__(kThreads) qk_rowsum_mfma_kernel(DotArgs a) {
  constexpr int NCH = ROUTE == 0 ? (W + 1) / 2 : W;  // products per 32 keys
  __shared__ v4i kt[NCH][64][2];                     // [product][key][half]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t bh = blockIdx.y, base = bh * a.N;
  const int qi = blockIdx.x * kBM + wave * 32 + li;
  v4i qop[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (ROUTE == 0) {
      const int word = 2 * c + lh;
      const uint32_t wq = (qi < a.N && word < W) ? a.qbits[(base + qi) * a.W + word] : 0u;
      qop[c] = expand_signs_fp4(wq, fp4_magnitude(word_valid(a.d, word)));
    } else {
      const uint32_t wq = qi < a.N ? a.qbits[(base + qi) * a.W + c] : 0u;
      qop[c] = expand_signs_i8(wq >> (16 * lh), half_valid(a.d, c, lh));
    }
  }
  v16f accf = v16f{};
  v16i acci = v16i{};
  for (int k0 = 0; k0 < a.N; k0 += 64) {
    __syncthreads();  // the previous tile is read
    for (int e = threadIdx.x; e < NCH * 128; e += kThreads) {
      const int c = e >> 7, key = (e >> 1) & 63, h = e & 1, kr = k0 + key;
      if (ROUTE == 0) {
        const int word = 2 * c + h;
        const uint32_t wk = (kr < a.N && word < W) ? a.kbits[(base + kr) * a.W + word] : 0u;
        kt[c][key][h] = expand_signs_fp4(wk, kr < a.N ? fp4_magnitude(word_valid(a.d, word)) : 0u);
      } else {
        const uint32_t wk = kr < a.N ? a.kbits[(base + kr) * a.W + c] : 0u;
        kt[c][key][h] = expand_signs_i8(wk >> (16 * h), kr < a.N ? half_valid(a.d, c, h) : 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const v4i kop = kt[c][32 * blk + li][lh];
        if (ROUTE == 0)
          accf = mfma_signs_32x32x64(kop, qop[c], accf);
        else
          acci = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qop[c], acci, 0, 0, 0);
      }
  }
  // each register holds an exact integer below 2^24; add them as integers
  int sum = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) sum += ROUTE == 0 ? static_cast<int>(accf[r]) : acci[r];
  sum += __shfl_xor(sum, 32, 64);
  if (lh == 0 && qi < a.N) a.dots[base + qi] = sum;
}

// Lane = query (64 a wave); the key words are wave-uniform, so they come in
// through scalar loads and every pair costs W v_xor + W v_bcnt.
template <int W>
__global__ void __launch_bounds__(kThreads) qk_rowsum_valu_kernel(DotArgs a) {
  const int64_t bh = blockIdx.y, base = bh * a.N;
  const int qi = blockIdx.x * kThreads + threadIdx.x;
  uint32_t q[W];
#pragma unroll
  for (int w = 0; w < W; ++w) q[w] = qi < a.N ? a.qbits[(base + qi) * W + w] : 0u;
  uint32_t ham = 0;
  const uint32_t* kb = a.kbits + base * W;
  for (int j = 0; j < a.N; ++j)
#pragma unroll
    for (int w = 0; w < W; ++w) ham += __popc(q[w] ^ kb[j * W + w]);
  if (qi < a.N) a.dots[base + qi] = a.N * a.d - 2 * static_cast<int>(ham);
}

__global__ void __launch_bounds__(kThreads) qk_dot_valu_kernel(DotArgs a) {
  const int j = blockIdx.x * kThreads + threadIdx.x;
  const int i = blockIdx.y;
  const int64_t bh = blockIdx.z;
  if (j >= a.N) return;
  const uint32_t* q = a.qbits + (bh * a.N + i) * a.W;
  const uint32_t* k = a.kbits + (bh * a.N + j) * a.W;
  int ham = 0;
  for (int w = 0; w < a.W; ++w) ham += __popc(q[w] ^ k[w]);
  a.dots[(bh * a.N + i) * a.N + j] = a.d - 2 * ham;
}

template <int W>
int launch_rowsum_w(const DotArgs& a, int route, hipStream_t s) {
  if (route == 1) {
    hipLaunchKernelGGL(qk_rowsum_valu_kernel<W>, dim3((a.N + kThreads - 1) / kThreads, static_cast<unsigned>(a.BH)),
                       dim3(kThreads), 0, s, a);
  } else if (route == 2) {
    hipLaunchKernelGGL((qk_rowsum_mfma_kernel<2, W>), dim3((a.N + kBM - 1) / kBM, static_cast<unsigned>(a.BH)),
                       dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((qk_rowsum_mfma_kernel<0, W>), dim3((a.N + kBM - 1) / kBM, static_cast<unsigned>(a.BH)),
                       dim3(kThreads), 0, s, a);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_qk_dot(const DotArgs& a, int route, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.rowsum) {
    switch (a.W) {
      case 1: return launch_rowsum_w<1>(a, route, s);
      case 2: return launch_rowsum_w<2>(a, route, s);
      case 3: return launch_rowsum_w<3>(a, route, s);
      case 4: return launch_rowsum_w<4>(a, route, s);
      case 5: return launch_rowsum_w<5>(a, route, s);
      case 6: return launch_rowsum_w<6>(a, route, s);
      case 7: return launch_rowsum_w<7>(a, route, s);
      case 8: return launch_rowsum_w<8>(a, route, s);
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  }
  if (route == 2) {
    const int nkb = (a.N + 31) / 32;
    const dim3 grid((nkb + 3) / 4, nkb, static_cast<unsigned>(a.BH));
    switch (a.W) {
      case 1: hipLaunchKernelGGL(qk_dot_i8_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
      case 2: hipLaunchKernelGGL(qk_dot_i8_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
      case 3: hipLaunchKernelGGL(qk_dot_i8_kernel<3>, grid, dim3(kThreads), 0, s, a); break;
      case 4: hipLaunchKernelGGL(qk_dot_i8_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
      case 5: hipLaunchKernelGGL(qk_dot_i8_kernel<5>, grid, dim3(kThreads), 0, s, a); break;
      case 6: hipLaunchKernelGGL(qk_dot_i8_kernel<6>, grid, dim3(kThreads), 0, s, a); break;
      case 7: hipLaunchKernelGGL(qk_dot_i8_kernel<7>, grid, dim3(kThreads), 0, s, a); break;
      case 8: hipLaunchKernelGGL(qk_dot_i8_kernel<8>, grid, dim3(kThreads), 0, s, a); break;
      default: return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
  }
  if (route == 1) {
    const dim3 grid((a.N + kThreads - 1) / kThreads, a.N, static_cast<unsigned>(a.BH));
    hipLaunchKernelGGL(qk_dot_valu_kernel, grid, dim3(kThreads), 0, s, a);
    return static_cast<int>(hipGetLastError());
  }
  const int nkb = (a.N + 31) / 32;
  const dim3 grid((nkb + 3) / 4, nkb, static_cast<unsigned>(a.BH));
  switch ((a.d + 63) / 64) {
    case 1: hipLaunchKernelGGL(qk_dot_mfma_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(qk_dot_mfma_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(qk_dot_mfma_kernel<3>, grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(qk_dot_mfma_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace ba
