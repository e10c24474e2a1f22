// Internal declarations shared by the host layer and the kernels.
#pragma once

#include <stdint.h>

#include "ba_device.h"

namespace ba {

// Tile sizes of the fused kernel: 4 waves x 32 queries, 64 keys per step.
constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
// N is padded per head to a multiple of this in every workspace array.
constexpr int kNAlign = 128;
// V^T rows in LDS: 64 keys + 8 bf16 of padding (144 bytes, 16-byte aligned,
// spreads rows over the LDS banks).
constexpr int kVtStride = 72;

// Zero rows on each side of the float32 bias rows in the workspace.
constexpr int kBiasPadRows = 8;
// Largest bias window (floats) the table-row path stages per key tile
// (8 KiB: two 1 KiB copy pieces per wave); covers grids up to 128 wide.
constexpr int kMaxWindowFloats = 2048;
// Dense-bias tile the fused kernel stages per key tile: 128 queries x 64 keys
// of bf16 (16 KiB, as floats).
constexpr int kDenseTileFloats = kBM * kBN / 2;

// Tokens per prologue block (one key tile).
constexpr int kPackTok = 64;

// Standalone sign pack of one tensor (ba_pack_signs).
struct PackJob {
  const uint16_t* x;  // bf16 [BH][N][d]
  uint32_t* bits;     // [BH][N][W]
  float* alpha;       // [BH][N]
  int64_t BH;
  int N, d, W;
};

// Keys and values of one forward, one 64-token tile of one (b, h) per block.
// Where token n of head (b, h) of a bf16 [B,H,N,d]-shaped view starts, in
// elements: b * sb + h * sh + n * sn (channels are contiguous).
struct Strides {
  int64_t sb, sh, sn;
};

__host__ __device__ inline int64_t token_offset(const Strides& s, int64_t b, int64_t h, int64_t n) {
  return b * s.sb + h * s.sh + n * s.sn;
}

struct KvJob {
  const uint16_t* k;  // bf16, strides ks
  const uint16_t* v;  // bf16, strides vs
  uint32_t* kop;      // fp4 key operands [BH][Npad/64][NCH][64][2][4]
  float* alpha;       // key scales [BH][Npad] (nullptr: not written)
  float* alpha_max;   // largest key scale of each tile [BH][Npad/64]
  uint16_t* vt;       // bf16 [BH][Npad/64][dpad][64], see the prologue
  // 8-bit P.V (vq != nullptr, then vt is unused): value codes, written as
  // the fused kernel's int8 operand tiles, from the per-tile channel maxima
  // of a previous launch; the scales and the column sums of the codes.
  int8_t* vq;         // [BH][Npad/64][dpad][64], see the prologue
  const float* vpart; // [BH][Npad/64][dpad] max |v| of each tile and channel
  float* vscale;      // [BH][dpad] max |v| / 127 (written by tile 0)
  int* vcsum;         // [BH][dpad] sum of the codes over the keys (atomic adds)
  // backward: the signs of the tile's tokens as +/-1 bf16 in the V^T layout
  // (nullptr: not written)
  uint16_t* kst;      // [BH][Npad/64][dpad][64]
  // backward: the largest |v| of each tile (nullptr: not written)
  float* vmax;        // [BH][Npad/64]
  // the values' rows as they are, contiguous [BH][Npad][d], zero past N
  // (nullptr: not written); with vt, vq, vmax and vnat all nullptr the
  // values are not read at all
  uint16_t* vnat;
  Strides ks, vs;
  int64_t BH;
  int H, N, Npad, d, W, nch, dpad;
  // the pipelined kernel's key-scale operands, per 64-token tile the words
  // w0 w1 of scale_split_a of each token (8 bytes each), then its w2 (nullptr:
  // not written)
  uint32_t* aks;      // [BH][Npad/64][192]
};

// Per-tile channel maxima of |V| for the 8-bit value codes, one 64-token
// tile of one (b, h) per block; tile 0 of each head also clears the head's
// column sums for the next launch.
struct VstatJob {
  const uint16_t* v;  // bf16, strides vs
  float* vpart;       // [BH][Npad/64][dpad]
  int* vcsum;         // [BH][dpad]
  Strides vs;
  int64_t BH;
  int H, N, Npad, d, dpad;
};

// Rows of the padded bias table one prologue block writes (one wave per
// row), and the 16-byte pieces per lane that cover a row: Lpad <= 320 floats
// (row mode has gw <= 128 in practice: 2gw-1+3 rounded to 16 mod 64 is 272).
constexpr int kBiasRowsPerBlock = 4;
constexpr int kBiasPieces = 5;

struct BiasJob {
  const uint16_t* table;  // bf16 [H][2gh-1][2gw-1]
  float* bias4;           // [H][2gh-1+2*kBiasPadRows][4][Lpad]
  float* row_max;         // [H][2gh-1]: max |entry| * log2(e) of each row
  int gh, gw, Lpad;
  int flip;               // 1: rows of the table flipped in both axes (the
                          // bias seen with queries and keys exchanged)
  int64_t nrows;          // H * (2gh-1+2*kBiasPadRows) padded rows
};

// Converts a caller's log-sum-exp ([BH][N], natural log) into the backward's
// row log2-sum-exp2 ([BH][Npad], 0 past N).  One thread per output entry.
struct LseJob {
  const float* in;
  float* out;
  int64_t BH;
  int N, Npad;
};

// The backward's delta_i = <dO_i, O_i> ([BH][Npad], 0 past N), from the
// contiguous [BH][N][d] dO and O, d % 16 == 0.  Two threads per row, each
// summing the products over its half of the channels (the 8-channel pieces
// 16 t + 8 half, in order of t), then the two halves added.
struct DeltaJob {
  const uint16_t* o;
  const uint16_t* dout;
  float* delta;
  int64_t BH;
  int N, Npad, d;
};

// Sums the workgroups' shares of the table gradient (see BwdArgs::dtpart):
// dtable[h][dyi][dx] = sum over b and query tiles qt of
// share[(b H + h) nqt + qt][dyi - row0(qt)][dx], row0 = (128 qt) / gw in
// table-row mode, 0 in table mode.  kDtEntries entries per block, kDtGroups
// threads per entry.
constexpr int kDtEntries = 32;
constexpr int kDtGroups = kThreads / kDtEntries;
struct DtReduceJob {
  const float* part;
  float* dtable;
  int B, H, nqt, gh, gw, prow, rows_mode;
};

// The relative-position table written out as a dense bias, for grids whose
// table rows fit neither the pipelined kernel's window nor LDS whole:
// out[h][i][j] = table[h][yi - yj + gh - 1][xi - xj + gw - 1] for i, j < N
// (token t at (t / gw, t % gw)), 0 for i or j in [N, Npad).  One block per
// (h, i) row.
struct ExpandJob {
  const uint16_t* table;  // bf16 [H][2gh-1][2gw-1]
  uint16_t* out;          // bf16 [H][Npad][Npad]
  int gh, gw, N, Npad;
};

// One launch runs the blocks of every job present (a job with 0 blocks is
// absent), in this order: pack, key/value tiles, bias rows, value
// statistics, the second bias rows, the table-gradient reduction, the
// log-sum-exp conversion, the dense expansion of a table.
struct PrologueArgs {
  PackJob pack;
  int64_t pack_blocks;
  KvJob kv;
  int64_t kv_blocks;
  BiasJob bias;
  int64_t bias_blocks;
  VstatJob vstat;
  int64_t vstat_blocks;
  BiasJob bias2;          // a second bias-row job (the flipped rows of the backward)
  int64_t bias2_blocks;
  DtReduceJob dtr;
  int64_t dtr_blocks;
  LseJob lsej;
  int64_t lse_blocks;
  DeltaJob delta;
  int64_t delta_blocks;
  ExpandJob expand;
  int64_t expand_blocks;
  int lds;  // dynamic LDS bytes per block
};

// Dynamic LDS the prologue needs for head dim d.
int prologue_lds(int d, bool kv);

int launch_prologue(const PrologueArgs& a, void* stream);

// kBiasRows / kBiasTable: a relative-position table; kBiasDense: one bf16
// value per (query, key) of each head (and batch entry).
enum BiasMode { kBiasNone = 0, kBiasRows = 1, kBiasTable = 2, kBiasDense = 3 };

struct FwdArgs {
  const uint16_t* q;       // bf16 queries (strides qs), packed in the kernel
  const uint32_t* kop;     // [BH][Npad/64][NCH][64 keys][2][4]: the fp4 +/-1
                           // operand dwords of each key, in LDS tile order
  const float* alpha_k;    // [BH][Npad]
  const uint16_t* vt;      // [BH][Npad/64][dpad][64] (slot order, swizzled)
  const float* bias4;      // kBiasRows: [H][2gh-1+2*kBiasPadRows][4][Lpad]
  const float* bias_row_max;  // kBiasRows: [H][2gh-1], max |b| log2e per row
  const float* kmax_blk;   // [BH][Npad/64] max alpha_k per 64-token block
  const uint32_t* aks;     // pipelined kernel: [BH][Npad/64][192] scale_split_a(alpha_k), see KvJob
  const uint16_t* table;   // kBiasTable: bf16 [H][2gh-1][2gw-1]
  const uint16_t* dense;   // kBiasDense: bias(b, h, i, j) at b*dsb + h*dsh + i*dld + j
  int64_t dsb, dsh, dld;
  int dense_shared;        // kBiasDense: 1 when dsb == 0 and B > 1
  const int8_t* vq;        // 8-bit P.V: value code tiles [BH][Npad/64][dpad][64]
  const float* vscale;     // 8-bit P.V: [BH][dpad] value scales
  const int* vcsum;        // 8-bit P.V: [BH][dpad] column sums of the codes
  uint16_t* o;             // bf16 output (strides os)
  float* lse;              // optional [BH][Npad]: mrow + log2(row sum), the
                           // logits' log2-sum-exp2 (for the backward pass)
  float* lse_out;          // optional [B*H][N]: the same in natural-log units,
                           // ln sum_j exp(S_ij) (the caller's copy)
  Strides qs, os;
  int B, H, N, Npad, d, W, dpad;
  int gh, gw, Lpad;
  int win_rows;            // kBiasRows: rows of the per-tile bias window
  float qscale;            // softmax scale * log2(e) (kBiasDense: softmax scale)
  int nqt;                 // query tiles per head
  int nwg;                 // workgroups
  int xcd_remap;           // 1: spread consecutive heads over the 8 XCDs
  int dyn_lds;             // dynamic LDS bytes per workgroup (table and/or padding)
  // the one-launch short-N kernel reads K and V itself (strides ks, vs)
  const uint16_t* k;
  const uint16_t* v;
  Strides ks, vs;
  int table_flip;          // kBiasTable: read the table flipped in both axes
  int prio_balance;        // 1: lower the wave priority over the last keys
                           // (every workgroup of the grid is resident at once)
};

// LDS bytes of the fused kernel: the bias table (table mode, dynamic) and
// the static tile buffers.
int fwd_table_lds(const FwdArgs& a, int mode);
int fwd_static_lds(int dpad, int mode);

// Waves per SIMD the fused kernel's register budget allows: 3 for up to 3
// accumulator blocks (32 output channels each, plus one when d % 32 == 0),
// 2 for up to 5, else 1.
// Waves per SIMD the general kernel's register budget is sized for, from
// its accumulator blocks nb and its 64-channel QK chunks nch: three blocks
// fit 168 registers with one chunk and not with two (d in (64, 96)), five
// fit 256 with two chunks and not with three (d in (128, 160)).
constexpr int fwd_waves_for_blocks(int nb, int nch = 1) {
  return (nb <= 3 && nch == 1) ? 3 : ((nb <= 5 && nch <= 2) ? 2 : 1);
}
int fwd_waves_per_simd(int dpad, int d);

// Launch the fused kernel (template selected from d and the bias mode).
int launch_attention(const FwdArgs& a, int mode, void* stream);
// The one-launch kernel for short sequences (no prologue): N <= 256,
// d in {32, 64}, table or no bias; reads a.k, a.v.
bool small_supported(int64_t N, int d, int mode);
int small_static_lds(int cb, int mode);
int launch_attention_small(const FwdArgs& a, int mode, void* stream);
// The fused kernel of the 8-bit P.V forward (d <= 128; no dense bias).
int launch_attention_int8(const FwdArgs& a, int mode, void* stream);
// The pipelined fused kernel (flash.hip): d in {32, 64, 72, 128}, table rows or
// no bias; reads V in its natural layout from a.v (strides a.vs), so the
// prologue writes no V^T for it.  win_rows * 4 * Lpad floats of bias window
// per key tile must fit its buffers.
bool flash_supported(int d, int mode, int win_rows, int Lpad);
int flash_static_lds(int d, int mode);
int flash_waves_per_simd(int d);
int launch_flash(const FwdArgs& a, int mode, void* stream);

// Backward pass (d in {32, 64, 128}; table-row, table or no bias).  One
// kernel, two roles: kRoleQ (lane = query; dq, delta, table gradient) and
// kRoleKV (lane = key; dk, dv).  f describes the row side (f.q: the lanes'
// tokens) and the column side (f.kop, f.alpha_k, f.kmax_blk, the bias) as
// the forward's arguments do.
enum BwdRole { kRoleQ = 0, kRoleKV = 1 };
struct BwdArgs {
  FwdArgs f;
  const uint16_t* xrow;    // [BH][N][d] the lanes' dP operand rows: dO (kRoleQ) or V (kRoleKV)
  const uint16_t* ynat;    // [BH][N][d] natural column tiles: V (kRoleQ) or dO (kRoleKV)
  const uint16_t* zt;      // [BH][Npad/64][dpad][64]: K signs (kRoleQ) or dO^T (kRoleKV)
  const uint16_t* zt2;     // [BH][Npad/64][dpad][64]: Q signs (kRoleKV)
  float* lse;              // [BH][Npad] log2-sum-exp2 of the query rows
  float* delta;            // [BH][Npad] <dO_i, O_i> (a prologue job, DeltaJob)
  float* out1;             // [BH][N][d] float32: dq (kRoleQ) or dk (kRoleKV)
  float* out2;             // kRoleKV: [BH][N][d] float32 dv
  float* dtable;           // kRoleQ: nullptr = no table gradient, else non-null (see dtpart)
  const float* vmax;       // kRoleQ, table mode with dtable: [BH][Npad/64] largest |v|
                           // of each key tile (the bound of the fixed-point sums)
  float* dtpart;           // kRoleQ: each workgroup's share of the table gradient,
                           // [B*H*nqt][prow][2gw-1]: rows dy from yq_lo - gh + 1
                           // (table rows) or the whole table (table mode, prow = 2gh-1)
  int prow;                // rows of one share
  float scale;             // the softmax scale
};
int bwd_static_lds(int role, int dpad, int mode);
int launch_backward(const BwdArgs& a, int role, int mode, void* stream);

struct DotArgs {
  const uint32_t* qbits;  // [BH][N][W]
  const uint32_t* kbits;  // [BH][N][W]
  int32_t* dots;          // [BH][N][N], or [BH][N] row sums
  int64_t BH;
  int N, d, W;
  int rowsum;             // 1: dots[bh][i] = sum_j D_ij
};

int launch_qk_dot(const DotArgs& a, int route, void* stream);

}  // namespace ba
