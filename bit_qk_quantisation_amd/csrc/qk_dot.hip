// QK integer dots D_ij = <sign q_i, sign k_j> for every pair: the check hook
// for the similarity step of the BinaryAttention kernel ("XNOR y popcount",
// "Representaciones Binarias Escaladas").
//
// Route BA_ROUTE_MFMA_FP4 runs exactly the device code of the fused kernel
// (expand_signs_fp4 + mfma_signs_32x32x64).  Route BA_ROUTE_VALU_POPCOUNT
// takes d - 2 popcount(q XOR k) on the packed words with v_xor/v_bcnt.
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

int launch_qk_dot(const DotArgs& a, int route, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
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
