// Host side of libbinattn.so: argument validation, workspace layout, kernel
// selection and launches.  See include/binattn.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ba_internal.h"
#include "binattn.h"

namespace {

thread_local char g_err[512] = "";

ba_status fail(ba_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int64_t kMaxTokens = (int64_t{1} << 31) - 1;

ba_status check_dims(int64_t B, int64_t H, int64_t N, int d) {
  if (B < 1 || H < 1 || N < 1) return fail(BA_ERR_SHAPE, "B, H and N must be >= 1 (got %lld, %lld, %lld)",
                                           (long long)B, (long long)H, (long long)N);
  if (d < 8 || d > 256 || d % 8 != 0)
    return fail(BA_ERR_UNSUPPORTED, "head dim d=%d unsupported (need 8 <= d <= 256, d %% 8 == 0)", d);
  if (B > kMaxTokens / H || B * H > kMaxTokens / round_up(N, ba::kNAlign))
    return fail(BA_ERR_SHAPE, "B*H*N too large (must stay below 2^31 tokens)");
  return BA_OK;
}

// Largest number of bias-table rows one (query tile, key tile) pair needs.
int window_rows(int64_t N, int gw) {
  const int64_t nqt = round_up(N, ba::kNAlign) / ba::kBM;
  const int64_t nkt = (N + ba::kBN - 1) / ba::kBN;
  int qspan = 0, kspan = 0;
  for (int64_t t = 0; t < nqt; ++t) {
    const int64_t q0 = t * ba::kBM;
    const int s = static_cast<int>((q0 + ba::kBM - 1) / gw - q0 / gw);
    if (s > qspan) qspan = s;
  }
  for (int64_t t = 0; t < nkt; ++t) {
    const int64_t k0 = t * ba::kBN;
    const int s = static_cast<int>((k0 + ba::kBN - 1) / gw - k0 / gw);
    if (s > kspan) kspan = s;
  }
  return qspan + kspan + 1;
}

// Floats per copy of a bias row: 2gw-1 entries + 3 of shift slack, rounded
// up to 16 (mod 64), so that the four shifted copies start 16 banks apart and
// 16 lanes reading 4 consecutive entries each never share a bank.
int64_t row_pad(int gw) {
  int64_t l = round_up(2 * static_cast<int64_t>(gw) - 1 + 3, 4);
  while (l % 64 != 16) l += 4;
  return l;
}

// Any other grid: the prologue writes the table out as a dense bias
// [H][Npad][Npad] in the workspace, which the dense-bias kernel reads.  Not a
// kernel mode: the plan turns it into kBiasDense.
constexpr int kModeExpand = 4;

// How the fused kernel reads the bias: table rows staged per key tile (grid
// width a multiple of 32, window small enough for the tile prefetch), the
// whole table in LDS (small tables), the table expanded into a dense bias
// (every other grid, up to 46336 tokens: the dense kernel addresses one
// head's bias with 32-bit offsets), or no bias.  -1: unsupported.
int choose_mode(bool has_bias, int gh, int gw, int64_t N) {
  if (!has_bias) return ba::kBiasNone;
  if (gw % 32 == 0 && window_rows(N, gw) > 0 && window_rows(N, gw) <= ba::kBiasPadRows &&
      window_rows(N, gw) * 4 * row_pad(gw) <= ba::kMaxWindowFloats && row_pad(gw) <= 64 * ba::kBiasPieces)
    return ba::kBiasRows;
  if (static_cast<int64_t>(2 * gh - 1) * (2 * gw - 1) * 4 <= 48 * 1024) return ba::kBiasTable;
  const int64_t npad = round_up(N, ba::kNAlign);
  if ((npad * npad + npad) * 2 < (int64_t{1} << 32)) return kModeExpand;
  return -1;
}

// Byte offsets of the workspace sections of ba_attention_fwd.
struct Layout {
  int64_t Npad, W, dpad, Lpad;
  int64_t kop, alpha_k, kmax, vt, vq, vpart, vscale, vcsum, bias4, rowmax, vnat, aks, expand, total;
  int mode;
  bool flash_prepared;  // the prepared forward runs the pipelined kernel on vnat
  bool no_vt;           // compact layout without V^T: only the pipelined kernel can run on it
};

// Whether the prepared forward (ba_attention_prepare + _fwd_prepared) runs
// the pipelined kernel: the kernel takes the shape, and the whole forward
// would not take the one-launch kernel (the pair then equals
// ba_attention_fwd bit for bit in every case).
bool prepared_flash(int64_t N, int d, int mode, int gw) {
  if (ba::small_supported(N, d, mode)) return false;
  const int win = mode == ba::kBiasRows ? window_rows(N, gw) : 0;
  return ba::flash_supported(d, mode, win, mode == ba::kBiasRows ? static_cast<int>(row_pad(gw)) : 0);
}

// int8pv: the 8-bit P.V forward, whose values are int8 code tiles with
// per-channel scales instead of the bf16 V^T copy.
// compact: the layout of ba_attention_fwd_static, which holds only what the
// whole forward reads: no V^T when the pipelined kernel runs (it reads V in
// place) and no natural copy of V (only the prepared forward uses one).
Layout layout(int64_t B, int64_t H, int64_t N, int d, bool has_bias, int gh, int gw, bool int8pv = false,
              bool compact = false) {
  Layout L{};
  L.Npad = round_up(N, ba::kNAlign);
  L.W = (d + 31) / 32;
  L.dpad = 32 * ((d + 31) / 32);
  L.mode = choose_mode(has_bias, gh, gw, N);
  L.Lpad = (L.mode == ba::kBiasRows) ? row_pad(gw) : 0;
  const int64_t BH = B * H;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.kop = take(BH * L.Npad * ((L.W + 1) / 2) * 32);  // fp4 key operands: 32 B per 64 channels
  L.alpha_k = take(BH * L.Npad * 4);
  L.kmax = take(BH * (L.Npad / 64) * 4);
  const bool rows0 = L.mode == ba::kBiasRows;
  const bool whole_flash = compact && !int8pv && L.mode >= 0 &&
                           ba::flash_supported(d, L.mode, rows0 ? window_rows(N, gw) : 0, static_cast<int>(L.Lpad));
  L.no_vt = whole_flash;
  L.vt = take((int8pv || whole_flash) ? 0 : BH * L.dpad * L.Npad * 2);
  L.vq = take(int8pv ? BH * L.dpad * L.Npad : 0);
  L.vpart = take(int8pv ? BH * (L.Npad / ba::kPackTok) * L.dpad * 4 : 0);
  L.vscale = take(int8pv ? BH * L.dpad * 4 : 0);
  L.vcsum = take(int8pv ? BH * L.dpad * 4 : 0);
  const bool rows = L.mode == ba::kBiasRows;
  L.bias4 = take(rows ? H * (2 * gh - 1 + 2 * ba::kBiasPadRows) * 4 * L.Lpad * 4 : 0);
  L.rowmax = take(rows ? H * (2 * gh - 1) * 4 : 0);
  // the values' natural rows, for the prepared forward's pipelined kernel
  L.flash_prepared = !int8pv && !compact && L.mode >= 0 && prepared_flash(N, d, L.mode, gw);
  L.vnat = take(L.flash_prepared ? BH * L.Npad * d * 2 : 0);
  // the pipelined kernel's key-scale operands (12 bytes per key)
  const bool flash_shape = !int8pv && L.mode >= 0 &&
                           ba::flash_supported(d, L.mode, rows0 ? window_rows(N, gw) : 0, static_cast<int>(L.Lpad));
  L.aks = take(flash_shape ? BH * L.Npad * 12 : 0);
  // the table written out as a dense bias, shared by the batch
  L.expand = take(L.mode == kModeExpand ? H * L.Npad * L.Npad * 2 : 0);
  L.total = off;
  return L;
}

ba_status hip_fail(int err, const char* what) {
  return fail(BA_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(err)));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// ---- strided [B,H,N,d] views -------------------------------------------------

ba::Strides contiguous_strides(int64_t H, int64_t N, int d) { return ba::Strides{H * N * d, N * d, d}; }

constexpr int64_t kMaxStride = int64_t{1} << 40;  // elements
constexpr int64_t kMaxSpan = int64_t{1} << 50;

// Checks one view's strides (non-negative, at most 2^40, multiples of 8 so
// that every row stays 16-byte aligned) and returns the number of bytes from
// its first to one past its last element, or -1.
int64_t view_span_bytes(const ba::Strides& s, int64_t B, int64_t H, int64_t N, int d) {
  const int64_t st[3] = {s.sb, s.sh, s.sn}, ext[3] = {B, H, N};
  int64_t span = d;
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0 || st[i] > kMaxStride || st[i] % 8 != 0) return -1;
    if (ext[i] > 1 && st[i] > (kMaxSpan - span) / (ext[i] - 1)) return -1;
    span += st[i] * (ext[i] - 1);
  }
  return span * 2;
}

// True when no element of the view belongs to two (b, h, n) rows: taken in
// order of increasing stride, each dimension's stride must step past
// everything the smaller ones reach.  Sufficient, not necessary; output views
// must pass it so that no two rows are written to the same place.
bool rows_disjoint(const ba::Strides& s, int64_t B, int64_t H, int64_t N, int d) {
  int64_t st[3] = {s.sb, s.sh, s.sn}, ext[3] = {B, H, N};
  for (int i = 1; i < 3; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      std::swap(st[j], st[j - 1]);
      std::swap(ext[j], ext[j - 1]);
    }
  int64_t reach = d;
  for (int i = 0; i < 3; ++i) {
    if (ext[i] <= 1) continue;
    if (st[i] < reach) return false;
    reach += st[i] * (ext[i] - 1);
  }
  return true;
}

// LDS bytes per compute unit on gfx950 (also the most one workgroup may use),
// and the allocation granule.
constexpr int kMaxLds = 160 * 1024;
constexpr int kLdsGranule = 512;

// Compute units of the current device, read once per device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// A second stream per device, on which the backward's key role runs beside
// the query role, with the events that fork it from the caller's stream and
// join it back.  Default priority, created on
// the device's first backward call and kept until the process ends.  The
// mutex spans fork to join, so calls from several host threads cannot mix
// their event records.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

// The side stream for work on `stream`, or nullptr when `stream` is not on
// the current device or creating the stream or its events failed (the caller
// then stays on one stream).  Call with g_side_mu held.
SideStream* side_stream_for(void* stream) {
  int dev = 0;
  hipDevice_t sdev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess || sdev != dev) return nullptr;
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (f) (void)hipEventDestroy(f);
      (void)hipStreamDestroy(s);
      return nullptr;
    }
    ss.s = s;
    ss.fork = f;
    ss.join = j;
  }
  return &ss;
}

// Dynamic LDS of the fused kernel: the bias table (table mode), raised when
// needed so that at most ceil(nwg / CUs) workgroups fit on one compute unit.
// With about k workgroups per unit in the grid, letting a unit take k+1 of
// them leaves others with k-1, and the busiest units set the time.
int fused_dynamic_lds(int static_lds, int table_lds, int64_t nwg) {
  int dyn = table_lds;
  const int cus = device_cus();
  if (cus > 0) {
    const int64_t k = (nwg + cus - 1) / cus;
    if (k >= 1 && k <= 4) {
      // more than kMaxLds / (k + 1) bytes each keeps the (k+1)-th out
      const int need = (kMaxLds / static_cast<int>(k + 1) / kLdsGranule + 1) * kLdsGranule;
      if (static_lds + dyn < need && need * k <= kMaxLds && need <= 64 * 1024) dyn = need - static_lds;
    }
  }
  return dyn;
}

// ---- backward -------------------------------------------------------------
// Workspace of ba_attention_bwd: the forward's sections, then (256-byte
// aligned, in this order) the K signs transposed, the forward output, the
// rows' log2-sum-exp2 and delta, the Q operand tiles, Q scales and their
// tile maxima, dO^T, the Q signs transposed, and the flipped bias rows.
struct BwdLayout {
  Layout fwd;
  int64_t kst, obuf, lse, delta, qop, alpha_q, qmax, dot, qst, bias4f, rowmaxf, vmax, dtpart, total;
  int prow;  // rows of one workgroup's share of the table gradient
};

// Largest number of grid rows, minus one, that a 128-query tile spans.
int query_span(int64_t N, int gw) {
  int qspan = 0;
  for (int64_t q0 = 0; q0 < round_up(N, ba::kNAlign); q0 += ba::kBM) {
    const int sp = static_cast<int>((q0 + ba::kBM - 1) / gw - q0 / gw);
    if (sp > qspan) qspan = sp;
  }
  return qspan;
}

BwdLayout bwd_layout(int64_t B, int64_t H, int64_t N, int d, bool has_bias, int gh, int gw) {
  BwdLayout L{};
  L.fwd = layout(B, H, N, d, has_bias, gh, gw);
  const int64_t BH = B * H, Npad = L.fwd.Npad, dpad = L.fwd.dpad, W = L.fwd.W;
  int64_t off = L.fwd.total;
  auto take = [&](int64_t bytes) {
    const int64_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.kst = take(BH * Npad * dpad * 2);
  L.obuf = take(BH * N * d * 2);
  L.lse = take(BH * Npad * 4);
  L.delta = take(BH * Npad * 4);
  L.qop = take(BH * Npad * ((W + 1) / 2) * 32);
  L.alpha_q = take(BH * Npad * 4);
  L.qmax = take(BH * (Npad / 64) * 4);
  L.dot = take(BH * Npad * dpad * 2);
  L.qst = take(BH * Npad * dpad * 2);
  const bool rows = L.fwd.mode == ba::kBiasRows;
  L.bias4f = take(rows ? H * (2 * gh - 1 + 2 * ba::kBiasPadRows) * 4 * L.fwd.Lpad * 4 : 0);
  L.rowmaxf = take(rows ? H * (2 * gh - 1) * 4 : 0);
  // table mode: the largest |v| of each key tile, for the table gradient's
  // fixed-point scale
  L.vmax = take(L.fwd.mode == ba::kBiasTable ? BH * (Npad / ba::kPackTok) * 4 : 0);
  // the shares of the table gradient: table rows yq_lo .. yq_hi + gh - 1 of
  // each query tile (table-row mode), or the whole table (table mode)
  L.prow = rows ? gh + query_span(N, gw) : (has_bias ? 2 * gh - 1 : 0);
  L.dtpart = take(has_bias ? BH * (Npad / ba::kBM) * L.prow * (2 * static_cast<int64_t>(gw) - 1) * 4 : 0);
  L.total = off;
  return L;
}

ba_status check_bwd_dims(int64_t B, int64_t H, int64_t N, int d) {
  ba_status st = check_dims(B, H, N, d);
  if (st != BA_OK) return st;
  if (d != 32 && d != 64 && d != 128) return fail(BA_ERR_UNSUPPORTED, "the backward supports d in {32, 64, 128} (d = %d)", d);
  return BA_OK;
}

}  // namespace

extern "C" {

int ba_version(void) { return BA_VERSION; }

const char* ba_status_string(ba_status s) {
  switch (s) {
    case BA_OK: return "BA_OK";
    case BA_ERR_NULL: return "BA_ERR_NULL";
    case BA_ERR_SHAPE: return "BA_ERR_SHAPE";
    case BA_ERR_UNSUPPORTED: return "BA_ERR_UNSUPPORTED";
    case BA_ERR_ALIGN: return "BA_ERR_ALIGN";
    case BA_ERR_WORKSPACE: return "BA_ERR_WORKSPACE";
    case BA_ERR_HIP: return "BA_ERR_HIP";
  }
  return "BA_ERR_UNKNOWN";
}

const char* ba_last_error(void) { return g_err; }

int ba_pack_words(int d) { return d < 1 ? 0 : (d + 31) / 32; }

ba_status ba_pack_signs(const void* x, int64_t B, int64_t H, int64_t N, int d,
                        uint32_t* bits, float* alpha, void* stream) {
  if (!x || !bits || !alpha) return fail(BA_ERR_NULL, "x, bits and alpha must be non-NULL");
  ba_status st = check_dims(B, H, N, d);
  if (st != BA_OK) return st;
  if (!aligned16(x) || !aligned16(bits) || !aligned16(alpha))
    return fail(BA_ERR_ALIGN, "x, bits and alpha must be 16-byte aligned");
  ba::PrologueArgs p{};
  p.pack = ba::PackJob{static_cast<const uint16_t*>(x), bits, alpha, B * H, static_cast<int>(N), d, (d + 31) / 32};
  p.pack_blocks = (B * H * N + ba::kPackTok - 1) / ba::kPackTok;
  p.lds = ba::prologue_lds(d, false);
  if (p.pack_blocks > 0x7fffffff) return fail(BA_ERR_SHAPE, "problem too large");
  const int err = ba::launch_prologue(p, stream);
  if (err != 0) return hip_fail(err, "pack launch");
  return BA_OK;
}

size_t ba_workspace_bytes_int8pv(int64_t B, int64_t H, int64_t N, int d, int gh, int gw) {
  if (check_dims(B, H, N, d) != BA_OK || d > 128 || N > 65536) return 0;
  const bool has_bias = gh > 0 || gw > 0;
  if (has_bias && (gh < 1 || gw < 1 || static_cast<int64_t>(gh) * gw != N)) return 0;
  const Layout L = layout(B, H, N, d, has_bias, gh, gw, true);
  if (L.mode < 0 || L.mode == kModeExpand) return 0;
  return static_cast<size_t>(L.total);
}

size_t ba_workspace_bytes(int64_t B, int64_t H, int64_t N, int d, int gh, int gw) {
  if (check_dims(B, H, N, d) != BA_OK) return 0;
  const bool has_bias = gh > 0 || gw > 0;
  if (has_bias && (gh < 1 || gw < 1 || static_cast<int64_t>(gh) * gw != N)) return 0;
  const Layout L = layout(B, H, N, d, has_bias, gh, gw);
  if (L.mode < 0) return 0;
  return static_cast<size_t>(L.total);
}

}  // extern "C"

namespace {

// A dense bias: bias(b, h, i, j) at ptr + b*sb + h*sh + i*ld + j elements.
struct DenseBias {
  const void* ptr;
  int64_t sb, sh, ld;
};

// Everything one forward needs: validated sizes, workspace sections and the
// arguments of both kernels.
struct Plan {
  ba::FwdArgs f;
  ba::PrologueArgs p0;  // 8-bit P.V only: value statistics and bias rows, before p
  ba::PrologueArgs p;
  int mode;
  bool int8pv;
  bool flash;  // the pipelined kernel (natural V, no V^T in the prologue)
};

// Validates a forward request.  `kv` selects the checks of k and v (the
// prologue's inputs), `qo` those of q and o (the fused kernel's input and
// output).
// `strides` holds the (batch, head, token) element strides of q, k, v and o,
// in that order (12 values), or is NULL for contiguous [B,H,N,d] tensors.
// `dense` (or NULL) is a dense bias; it excludes a bias table.
ba_status make_plan(const void* q, const void* k, const void* v, bool kv, const void* bias, int gh, int gw,
                    int64_t B, int64_t H, int64_t N, int d, float scale, void* o, bool qo,
                    const int64_t* strides, const DenseBias* dense, void* workspace, size_t ws_bytes,
                    Plan* plan, bool int8pv = false, bool allow_flash = true, bool compact = false) {
  if (kv && (!k || !v)) return fail(BA_ERR_NULL, "k and v must be non-NULL");
  if (qo && (!q || !o)) return fail(BA_ERR_NULL, "q and o must be non-NULL");
  ba_status st = check_dims(B, H, N, d);
  if (st != BA_OK) return st;
  if (qo && (!std::isfinite(scale) || scale < 0.0f))
    return fail(BA_ERR_SHAPE, "scale must be finite and >= 0");
  if (bias) {
    if (gh < 1 || gw < 1 || static_cast<int64_t>(gh) * gw != N)
      return fail(BA_ERR_SHAPE, "with a bias table gh*gw must equal N (gh=%d gw=%d N=%lld)", gh, gw,
                  (long long)N);
  }
  if ((kv && (!aligned16(k) || !aligned16(v))) || (qo && (!aligned16(q) || !aligned16(o))) ||
      (bias && !aligned16(bias)))
    return fail(BA_ERR_ALIGN, "q, k, v, o and bias must be 16-byte aligned");
  ba::Strides vs[4];  // q, k, v, o
  for (int t = 0; t < 4; ++t)
    vs[t] = strides ? ba::Strides{strides[3 * t], strides[3 * t + 1], strides[3 * t + 2]}
                    : contiguous_strides(H, N, d);
  int64_t span[4];
  static const char* const names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t) {
    span[t] = view_span_bytes(vs[t], B, H, N, d);
    if (span[t] < 0)
      return fail(BA_ERR_SHAPE, "%s strides (%lld, %lld, %lld) must be multiples of 8 in [0, 2^40] and span "
                  "at most 2^50 elements", names[t], (long long)vs[t].sb, (long long)vs[t].sh, (long long)vs[t].sn);
  }
  if (qo && !rows_disjoint(vs[3], B, H, N, d))
    return fail(BA_ERR_SHAPE, "o strides (%lld, %lld, %lld) let two output rows overlap", (long long)vs[3].sb,
                (long long)vs[3].sh, (long long)vs[3].sn);
  const size_t qb = span[0], kb = span[1], vb = span[2], ob = span[3];
  if (qo && (overlaps(o, ob, q, qb) || (kv && (overlaps(o, ob, k, kb) || overlaps(o, ob, v, vb)))))
    return fail(BA_ERR_SHAPE, "o must not overlap q, k or v");
  if (dense && qo) {
    if (bias) return fail(BA_ERR_SHAPE, "a dense bias and a bias table cannot be combined");
    if (!dense->ptr) return fail(BA_ERR_NULL, "bias must be non-NULL");
    if (!aligned16(dense->ptr)) return fail(BA_ERR_ALIGN, "bias must be 16-byte aligned");
    const int64_t st[3] = {dense->sb, dense->sh, dense->ld}, ext[3] = {B, H, N};
    int64_t bspan = N;  // elements from the first to one past the last
    for (int i = 0; i < 3; ++i) {
      if (st[i] < 0 || st[i] > kMaxStride || st[i] % 8 != 0)
        return fail(BA_ERR_SHAPE, "dense bias strides (%lld, %lld, %lld) must be multiples of 8 in [0, 2^40]",
                    (long long)dense->sb, (long long)dense->sh, (long long)dense->ld);
      if (ext[i] > 1 && st[i] > (kMaxSpan - bspan) / (ext[i] - 1))
        return fail(BA_ERR_SHAPE, "dense bias spans more than 2^50 elements");
      bspan += st[i] * (ext[i] - 1);
    }
    const int64_t npad = round_up(N, ba::kNAlign);
    if ((npad * dense->ld + npad) * 2 >= (int64_t{1} << 32))
      return fail(BA_ERR_UNSUPPORTED, "dense bias of one head must span less than 4 GiB ((N rounded up to 128) "
                  "* (ld + 1) * 2 bytes)");
    if (overlaps(o, ob, dense->ptr, static_cast<size_t>(bspan) * 2))
      return fail(BA_ERR_SHAPE, "o must not overlap the bias");
  }
  if (int8pv) {
    if (d > 128) return fail(BA_ERR_UNSUPPORTED, "the 8-bit P.V forward supports d <= 128 (d = %d)", d);
    if (N > 65536)
      return fail(BA_ERR_UNSUPPORTED, "the 8-bit P.V forward supports N <= 65536 (exact int32 sums), N = %lld",
                  (long long)N);
  }
  int mode = dense ? static_cast<int>(ba::kBiasDense) : choose_mode(bias != nullptr, gh, gw, N);
  if (mode < 0)
    return fail(BA_ERR_UNSUPPORTED,
                "bias grid %dx%d: the table rows do not fit the tile window, the table exceeds 48 KiB and its "
                "dense form would span 4 GiB or more per head", gh, gw);
  const bool expand = mode == kModeExpand;
  if (expand && int8pv)
    return fail(BA_ERR_UNSUPPORTED, "bias grid %dx%d: the 8-bit P.V forward takes table rows (gw %% 32 == 0) or "
                "tables of at most 48 KiB", gh, gw);
  const Layout L = layout(B, H, N, d, bias != nullptr, dense ? 0 : gh, dense ? 0 : gw, int8pv, compact);
  if (!workspace) return fail(BA_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(BA_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (ws_bytes < static_cast<size_t>(L.total))
    return fail(BA_ERR_WORKSPACE, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)L.total);
  if (qo && (overlaps(workspace, L.total, o, ob) || overlaps(workspace, L.total, q, qb)))
    return fail(BA_ERR_WORKSPACE, "workspace must not overlap q or o");
  if (kv && (overlaps(workspace, L.total, k, kb) || overlaps(workspace, L.total, v, vb)))
    return fail(BA_ERR_WORKSPACE, "workspace must not overlap k or v");
  if (bias && overlaps(workspace, L.total, bias, static_cast<size_t>(H * (2 * gh - 1) * (2 * gw - 1)) * 2))
    return fail(BA_ERR_WORKSPACE, "workspace must not overlap the bias table");

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const int64_t BH = B * H;
  DenseBias expanded{};
  if (expand) {  // the fused kernel reads the prologue's dense form of the table
    expanded = DenseBias{ws + L.expand, 0, L.Npad * L.Npad, L.Npad};
    dense = &expanded;
    mode = ba::kBiasDense;
  }
  ba::FwdArgs& f = plan->f;
  f = ba::FwdArgs{};
  f.q = static_cast<const uint16_t*>(q);
  f.kop = reinterpret_cast<const uint32_t*>(ws + L.kop);
  f.alpha_k = reinterpret_cast<const float*>(ws + L.alpha_k);
  f.vt = reinterpret_cast<const uint16_t*>(ws + L.vt);
  if (int8pv) {
    f.vq = reinterpret_cast<const int8_t*>(ws + L.vq);
    f.vscale = reinterpret_cast<const float*>(ws + L.vscale);
    f.vcsum = reinterpret_cast<const int*>(ws + L.vcsum);
  }
  f.bias4 = reinterpret_cast<const float*>(ws + L.bias4);
  f.bias_row_max = reinterpret_cast<const float*>(ws + L.rowmax);
  f.kmax_blk = reinterpret_cast<const float*>(ws + L.kmax);
  f.table = static_cast<const uint16_t*>(bias);
  if (dense) {
    f.dense = static_cast<const uint16_t*>(dense->ptr);
    f.dsb = dense->sb;
    f.dsh = dense->sh;
    f.dld = dense->ld;
    f.dense_shared = (dense->sb == 0 && B > 1) ? 1 : 0;
  }
  f.o = static_cast<uint16_t*>(o);
  f.qs = vs[0];
  f.os = vs[3];
  f.k = static_cast<const uint16_t*>(k);
  f.v = static_cast<const uint16_t*>(v);
  f.ks = vs[1];
  f.vs = vs[2];
  f.B = static_cast<int>(B);
  f.H = static_cast<int>(H);
  f.N = static_cast<int>(N);
  f.Npad = static_cast<int>(L.Npad);
  f.d = d;
  f.W = static_cast<int>(L.W);
  f.dpad = static_cast<int>(L.dpad);
  f.gh = gh;
  f.gw = gw;
  f.Lpad = static_cast<int>(L.Lpad);
  f.win_rows = (mode == ba::kBiasRows) ? window_rows(N, gw) : 0;
  f.qscale = dense ? scale : scale * ba::kLog2e;  // dense logits stay in natural units
  f.nqt = static_cast<int>(L.Npad / ba::kBM);
  const int64_t nwg = BH * f.nqt;
  if (nwg > 0x7fffffff) return fail(BA_ERR_SHAPE, "too many workgroups");
  f.nwg = static_cast<int>(nwg);
  f.xcd_remap = (f.nwg % 8 == 0) ? 1 : 0;
  // The pipelined kernel reads V in its natural layout: from the caller's v
  // in a whole forward, from the workspace copy ba_attention_prepare writes
  // for the prepared forward.  Its copies address one head's value rows with
  // 32-bit byte offsets.
  // ba_attention_prepare (kv, not qo) writes V^T (for the dense-bias
  // prepared forward and the other kernels) and, when the prepared forward
  // takes the pipelined kernel, the natural copy as well.
  const bool whole = kv && qo, prepared = qo && !kv, preparing = kv && !qo;
  bool flash = allow_flash && !dense && !int8pv && !preparing &&
               (prepared ? L.flash_prepared : ba::flash_supported(d, mode, f.win_rows, f.Lpad));
  if (flash && whole && (static_cast<int64_t>(L.Npad) * vs[2].sn + d) * 2 >= (int64_t{1} << 31)) flash = false;
  if (L.no_vt && !flash)
    return fail(BA_ERR_UNSUPPORTED, "the value rows span 2 GiB or more: this entry point cannot run the problem");
  uint16_t* vnat = reinterpret_cast<uint16_t*>(ws + L.vnat);
  uint32_t* aks = reinterpret_cast<uint32_t*>(ws + L.aks);
  f.aks = aks;
  if (flash) {
    if (whole) {
      f.v = static_cast<const uint16_t*>(v);
      f.vs = vs[2];
    } else {
      f.v = vnat;
      f.vs = ba::Strides{H * L.Npad * d, L.Npad * d, d};
    }
  }
  const int static_lds = flash ? ba::flash_static_lds(d, mode) : ba::fwd_static_lds(f.dpad, mode);
  const int table_lds = flash ? 0 : ba::fwd_table_lds(f, mode);
  if (static_lds + table_lds > kMaxLds) return fail(BA_ERR_UNSUPPORTED, "bias window does not fit in LDS");
  f.dyn_lds = fused_dynamic_lds(static_lds, table_lds, nwg);
  {
    const int cus = device_cus();
    const int per_wg = static_cast<int>(round_up(static_lds + f.dyn_lds, kLdsGranule));
    const int waves = flash ? ba::flash_waves_per_simd(d) : ba::fwd_waves_per_simd(f.dpad, d);
    const int resident = std::min(waves, kMaxLds / per_wg);
    f.prio_balance = (cus > 0 && nwg <= static_cast<int64_t>(cus) * resident) ? 1 : 0;
  }

  ba::PrologueArgs& p = plan->p;
  p = ba::PrologueArgs{};
  // the pipelined kernel takes the key scales only as matrix operands (aks)
  const bool scales_as_floats = !(flash && whole);
  p.kv = ba::KvJob{static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), const_cast<uint32_t*>(f.kop),
                   scales_as_floats ? const_cast<float*>(f.alpha_k) : nullptr, const_cast<float*>(f.kmax_blk),
                   flash ? nullptr : const_cast<uint16_t*>(f.vt),
                   nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                   (preparing && L.flash_prepared) ? vnat : nullptr,
                   vs[1], vs[2], BH, static_cast<int>(H), f.N, f.Npad, d, f.W, (f.W + 1) / 2, f.dpad,
                   (flash || (preparing && L.flash_prepared)) ? aks : nullptr};
  p.kv_blocks = BH * (L.Npad / ba::kPackTok);
  p.lds = ba::prologue_lds(d, true);
  // the 8-bit forward builds the bias rows in its first launch, beside the
  // value statistics the second launch needs
  plan->p0 = ba::PrologueArgs{};
  ba::PrologueArgs& pb = int8pv ? plan->p0 : p;
  if (mode == ba::kBiasRows) {
    const int64_t nrows = H * (2 * gh - 1 + 2 * ba::kBiasPadRows);
    pb.bias = ba::BiasJob{static_cast<const uint16_t*>(bias), const_cast<float*>(f.bias4),
                          const_cast<float*>(f.bias_row_max), gh, gw, f.Lpad, 0, nrows};
    pb.bias_blocks = (nrows + ba::kBiasRowsPerBlock - 1) / ba::kBiasRowsPerBlock;
  }
  if (int8pv) {
    float* vpart = reinterpret_cast<float*>(ws + L.vpart);
    int* vcsum = reinterpret_cast<int*>(ws + L.vcsum);
    pb.vstat = ba::VstatJob{static_cast<const uint16_t*>(v), vpart, vcsum, vs[2], BH, static_cast<int>(H),
                            f.N, f.Npad, d, f.dpad};
    pb.vstat_blocks = kv ? BH * (L.Npad / ba::kPackTok) : 0;
    pb.lds = f.dpad * 4;
    p.kv.vq = reinterpret_cast<int8_t*>(ws + L.vq);
    p.kv.vpart = vpart;
    p.kv.vscale = reinterpret_cast<float*>(ws + L.vscale);
    p.kv.vcsum = vcsum;
  }
  if (expand) {
    p.expand = ba::ExpandJob{static_cast<const uint16_t*>(bias), reinterpret_cast<uint16_t*>(ws + L.expand), gh, gw,
                             f.N, f.Npad};
    p.expand_blocks = kv ? H * L.Npad : 0;
  }
  const int64_t pblocks = p.kv_blocks + pb.bias_blocks + pb.vstat_blocks + p.expand_blocks;
  if (pblocks > 0x7fffffff) return fail(BA_ERR_SHAPE, "problem too large");
  plan->mode = mode;
  plan->int8pv = int8pv;
  plan->flash = flash;
  return BA_OK;
}

ba_status run_forward(const void* q, const void* k, const void* v, const void* bias, int gh, int gw, int64_t B,
                      int64_t H, int64_t N, int d, float scale, void* o, const int64_t* strides,
                      const DenseBias* dense, void* workspace, size_t ws_bytes, void* stream,
                      float* lse_out = nullptr, bool compact = false) {
  Plan plan;
  ba_status st = make_plan(q, k, v, true, bias, gh, gw, B, H, N, d, scale, o, true, strides, dense, workspace,
                           ws_bytes, &plan, false, true, compact);
  if (st != BA_OK) return st;
  if (lse_out) {
    const size_t lb = static_cast<size_t>(B * H * N) * 4, tb = static_cast<size_t>(B * H * N * d) * 2;
    if ((reinterpret_cast<uintptr_t>(lse_out) & 3u) != 0) return fail(BA_ERR_ALIGN, "lse must be 4-byte aligned");
    const void* others[4] = {q, k, v, o};
    for (const void* x : others)
      if (overlaps(lse_out, lb, x, tb)) return fail(BA_ERR_SHAPE, "lse must not overlap q, k, v or o");
    if (overlaps(lse_out, lb, workspace, ws_bytes)) return fail(BA_ERR_WORKSPACE, "lse overlaps the workspace");
    plan.f.lse_out = lse_out;
  }
  if (!dense && ba::small_supported(N, d, plan.mode)) {
    // short sequences: one launch, the keys and values packed in LDS
    ba::FwdArgs f = plan.f;
    const int sl = ba::small_static_lds(f.dpad / 32, plan.mode);
    f.dyn_lds = fused_dynamic_lds(sl, ba::fwd_table_lds(f, plan.mode), f.nwg);
    if (sl + f.dyn_lds <= kMaxLds) {
      const int err = ba::launch_attention_small(f, plan.mode, stream);
      if (err != 0) return hip_fail(err, "attention launch");
      return BA_OK;
    }
  }
  int err = ba::launch_prologue(plan.p, stream);
  if (err != 0) return hip_fail(err, "prologue launch");
  err = plan.flash ? ba::launch_flash(plan.f, plan.mode, stream) : ba::launch_attention(plan.f, plan.mode, stream);
  if (err != 0) return hip_fail(err, "attention launch");
  return BA_OK;
}

}  // namespace

extern "C" {

ba_status ba_attention_prepare(const void* k, const void* v, const void* bias, int gh, int gw, int64_t B,
                               int64_t H, int64_t N, int d, void* workspace, size_t ws_bytes, void* stream) {
  Plan plan;
  ba_status st = make_plan(nullptr, k, v, true, bias, gh, gw, B, H, N, d, 0.0f, nullptr, false, nullptr, nullptr,
                           workspace, ws_bytes, &plan);
  if (st != BA_OK) return st;
  const int err = ba::launch_prologue(plan.p, stream);
  if (err != 0) return hip_fail(err, "prologue launch");
  return BA_OK;
}

ba_status ba_attention_fwd_prepared(const void* q, const void* bias, int gh, int gw, int64_t B, int64_t H,
                                    int64_t N, int d, float scale, void* o, const void* workspace,
                                    size_t ws_bytes, void* stream) {
  Plan plan;
  ba_status st = make_plan(q, nullptr, nullptr, false, bias, gh, gw, B, H, N, d, scale, o, true, nullptr, nullptr,
                           const_cast<void*>(workspace), ws_bytes, &plan);
  if (st != BA_OK) return st;
  const int err = plan.flash ? ba::launch_flash(plan.f, plan.mode, stream) : ba::launch_attention(plan.f, plan.mode, stream);
  if (err != 0) return hip_fail(err, "attention launch");
  return BA_OK;
}

ba_status ba_attention_fwd_int8pv(const void* q, const void* k, const void* v, const void* bias, int gh, int gw,
                                  int64_t B, int64_t H, int64_t N, int d, float scale, void* o, void* workspace,
                                  size_t ws_bytes, void* stream) {
  Plan plan;
  ba_status st = make_plan(q, k, v, true, bias, gh, gw, B, H, N, d, scale, o, true, nullptr, nullptr, workspace,
                           ws_bytes, &plan, true);
  if (st != BA_OK) return st;
  int err = ba::launch_prologue(plan.p0, stream);
  if (err != 0) return hip_fail(err, "value statistics launch");
  err = ba::launch_prologue(plan.p, stream);
  if (err != 0) return hip_fail(err, "prologue launch");
  err = ba::launch_attention_int8(plan.f, plan.mode, stream);
  if (err != 0) return hip_fail(err, "attention launch");
  return BA_OK;
}

ba_status ba_attention_fwd_dense_bias_prepared(const void* q, const void* bias, int64_t bias_sb, int64_t bias_sh,
                                               int64_t bias_ld, int64_t B, int64_t H, int64_t N, int d,
                                               float scale, void* o, const void* workspace, size_t ws_bytes,
                                               void* stream) {
  Plan plan;
  const DenseBias dense{bias, bias_sb, bias_sh, bias_ld};
  ba_status st = make_plan(q, nullptr, nullptr, false, nullptr, 0, 0, B, H, N, d, scale, o, true, nullptr, &dense,
                           const_cast<void*>(workspace), ws_bytes, &plan);
  if (st != BA_OK) return st;
  const int err = ba::launch_attention(plan.f, plan.mode, stream);
  if (err != 0) return hip_fail(err, "attention launch");
  return BA_OK;
}

ba_status ba_attention_fwd(const void* q, const void* k, const void* v,
                           const void* bias, int gh, int gw,
                           int64_t B, int64_t H, int64_t N, int d, float scale,
                           void* o, void* workspace, size_t ws_bytes, void* stream) {
  return run_forward(q, k, v, bias, gh, gw, B, H, N, d, scale, o, nullptr, nullptr, workspace, ws_bytes, stream);
}

ba_status ba_attention_fwd_train(const void* q, const void* k, const void* v,
                                 const void* bias, int gh, int gw,
                                 int64_t B, int64_t H, int64_t N, int d, float scale,
                                 void* o, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (!lse) return fail(BA_ERR_NULL, "lse must be non-NULL");
  return run_forward(q, k, v, bias, gh, gw, B, H, N, d, scale, o, nullptr, nullptr, workspace, ws_bytes, stream,
                     lse);
}

ba_status ba_attention_fwd_strided(const void* q, const void* k, const void* v,
                                   const void* bias, int gh, int gw,
                                   int64_t B, int64_t H, int64_t N, int d, float scale,
                                   void* o, const int64_t* strides,
                                   void* workspace, size_t ws_bytes, void* stream) {
  if (!strides) return fail(BA_ERR_NULL, "strides must be non-NULL");
  return run_forward(q, k, v, bias, gh, gw, B, H, N, d, scale, o, strides, nullptr, workspace, ws_bytes, stream);
}

ba_status ba_attention_fwd_static(const void* q, const void* k, const void* v, const void* bias, int gh, int gw,
                                  int64_t B, int64_t H, int64_t N, int d, float scale, void* o, void* stream);

ba_status ba_attention_fwd_dense_bias(const void* q, const void* k, const void* v,
                                      const void* bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_ld,
                                      int64_t B, int64_t H, int64_t N, int d, float scale,
                                      void* o, const int64_t* strides,
                                      void* workspace, size_t ws_bytes, void* stream) {
  const DenseBias dense{bias, bias_sb, bias_sh, bias_ld};
  return run_forward(q, k, v, nullptr, 0, 0, B, H, N, d, scale, o, strides, &dense, workspace, ws_bytes, stream);
}

}  // extern "C"

namespace {

// The backward, with the forward recomputed (o_saved == nullptr) or with the
// caller's O and log-sum-exp from ba_attention_fwd_train.
ba_status run_backward(const void* q, const void* k, const void* v, const void* bias, int gh, int gw, int64_t B,
                       int64_t H, int64_t N, int d, float scale, const void* o_saved, const float* lse_saved,
                       const void* dout, float* dq, float* dk, float* dv, float* dtable, void* workspace,
                       size_t ws_bytes, void* stream) {
  ba_status st = check_bwd_dims(B, H, N, d);
  if (st != BA_OK) return st;
  if (!q || !dout || !dq || !dk || !dv) return fail(BA_ERR_NULL, "q, dout, dq, dk and dv must be non-NULL");
  if (!std::isfinite(scale) || scale < 0.0f) return fail(BA_ERR_SHAPE, "scale must be finite and >= 0");
  if (!aligned16(q)) return fail(BA_ERR_ALIGN, "q must be 16-byte aligned");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || (dtable && !aligned16(dtable)))
    return fail(BA_ERR_ALIGN, "dout, dq, dk, dv and dtable must be 16-byte aligned");
  const BwdLayout BL = bwd_layout(B, H, N, d, bias != nullptr, gh, gw);
  if (BL.fwd.mode == kModeExpand)
    return fail(BA_ERR_UNSUPPORTED, "bias grid %dx%d: the backward takes table rows (gw %% 32 == 0) or tables of at "
                "most 48 KiB", gh, gw);
  if (ws_bytes < static_cast<size_t>(BL.total))
    return fail(BA_ERR_WORKSPACE, "workspace too small: %zu < %lld bytes", ws_bytes, (long long)BL.total);
  // the forward's plan validates q, k, v, the bias and the first part of the workspace
  Plan fp;
  st = make_plan(q, k, v, true, bias, gh, gw, B, H, N, d, scale, nullptr, false, nullptr, nullptr, workspace,
                 ws_bytes, &fp, false, false);
  if (st != BA_OK) return st;
  if (!workspace) return fail(BA_ERR_WORKSPACE, "workspace is NULL");
  const size_t tb = static_cast<size_t>(B * H * N * d);
  const void* ins[4] = {q, k, v, dout};
  const void* outs[3] = {dq, dk, dv};
  // the backward writes all of its workspace, also the part past the forward's
  for (const void* i : ins)
    if (overlaps(i, tb * 2, workspace, BL.total))
      return fail(BA_ERR_WORKSPACE, "q, k, v and dout must not overlap the workspace");
  if (bias && overlaps(bias, static_cast<size_t>(H * (2 * gh - 1) * (2 * gw - 1)) * 2, workspace, BL.total))
    return fail(BA_ERR_WORKSPACE, "the bias table must not overlap the workspace");
  for (const void* o : outs) {
    for (const void* i : ins)
      if (overlaps(o, tb * 4, i, tb * 2)) return fail(BA_ERR_SHAPE, "gradients must not overlap the inputs");
    if (overlaps(o, tb * 4, workspace, BL.total)) return fail(BA_ERR_WORKSPACE, "gradients overlap the workspace");
  }
  if (overlaps(dq, tb * 4, dk, tb * 4) || overlaps(dq, tb * 4, dv, tb * 4) || overlaps(dk, tb * 4, dv, tb * 4))
    return fail(BA_ERR_SHAPE, "dq, dk and dv must not overlap");
  const int mode = fp.mode;
  const int64_t tcount = bias ? H * (2 * gh - 1) * (2 * gw - 1) : 0;
  if (dtable && !bias) return fail(BA_ERR_SHAPE, "dtable needs a bias table");
  if (dtable && overlaps(dtable, tcount * 4, workspace, BL.total))
    return fail(BA_ERR_WORKSPACE, "dtable overlaps the workspace");
  if (dtable) {
    // (dtable is written while the key role writes dk and dv)
    for (const void* o : outs)
      if (overlaps(dtable, tcount * 4, o, tb * 4)) return fail(BA_ERR_SHAPE, "dtable must not overlap dq, dk or dv");
    for (const void* i : ins)
      if (overlaps(dtable, tcount * 4, i, tb * 2)) return fail(BA_ERR_SHAPE, "dtable must not overlap the inputs");
    if (overlaps(dtable, tcount * 4, bias, tcount * 2)) return fail(BA_ERR_SHAPE, "dtable must not overlap the table");
  }
  const bool saved = o_saved != nullptr;
  if (saved) {
    if (!lse_saved) return fail(BA_ERR_NULL, "lse must be non-NULL");
    if (!aligned16(o_saved)) return fail(BA_ERR_ALIGN, "o must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse_saved) & 3u) != 0) return fail(BA_ERR_ALIGN, "lse must be 4-byte aligned");
    const size_t lb = static_cast<size_t>(B * H * N) * 4;
    for (const void* g : outs)
      if (overlaps(g, tb * 4, o_saved, tb * 2) || overlaps(g, tb * 4, lse_saved, lb))
        return fail(BA_ERR_SHAPE, "gradients must not overlap o or lse");
    if (dtable && (overlaps(dtable, tcount * 4, o_saved, tb * 2) || overlaps(dtable, tcount * 4, lse_saved, lb)))
      return fail(BA_ERR_SHAPE, "dtable must not overlap o or lse");
    if (overlaps(o_saved, tb * 2, workspace, BL.total) || overlaps(lse_saved, lb, workspace, BL.total))
      return fail(BA_ERR_WORKSPACE, "o and lse must not overlap the workspace");
  }

  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* obuf = reinterpret_cast<uint16_t*>(ws + BL.obuf);
  float* lse = reinterpret_cast<float*>(ws + BL.lse);
  float* delta = reinterpret_cast<float*>(ws + BL.delta);

  // 1. keys and values (with the K signs transposed), both bias-row orientations
  ba::PrologueArgs p1 = fp.p;
  p1.kv.kst = reinterpret_cast<uint16_t*>(ws + BL.kst);
  float* vmax = (mode == ba::kBiasTable && dtable) ? reinterpret_cast<float*>(ws + BL.vmax) : nullptr;
  p1.kv.vmax = vmax;
  if (mode == ba::kBiasRows) {
    p1.bias2 = p1.bias;
    p1.bias2.bias4 = reinterpret_cast<float*>(ws + BL.bias4f);
    p1.bias2.row_max = reinterpret_cast<float*>(ws + BL.rowmaxf);
    p1.bias2.flip = 1;
    p1.bias2_blocks = p1.bias_blocks;
  }
  // 2. the forward, keeping O and the rows' log2-sum-exp2
  ba::FwdArgs f = fp.f;
  f.o = obuf;
  f.os = contiguous_strides(H, N, d);
  f.lse = lse;
  // 3. queries and dO as the keys and values of a second prologue pass, and delta
  ba::PrologueArgs p3{};
  p3.kv = p1.kv;
  p3.kv.vmax = nullptr;  // dO's maxima are not needed
  p3.kv.k = static_cast<const uint16_t*>(q);
  p3.kv.v = static_cast<const uint16_t*>(dout);
  p3.kv.kop = reinterpret_cast<uint32_t*>(ws + BL.qop);
  p3.kv.alpha = reinterpret_cast<float*>(ws + BL.alpha_q);
  p3.kv.alpha_max = reinterpret_cast<float*>(ws + BL.qmax);
  p3.kv.vt = reinterpret_cast<uint16_t*>(ws + BL.dot);
  p3.kv.kst = reinterpret_cast<uint16_t*>(ws + BL.qst);
  p3.kv.ks = contiguous_strides(H, N, d);
  p3.kv.vs = contiguous_strides(H, N, d);
  p3.kv_blocks = p1.kv_blocks;
  p3.lds = p1.lds;
  if (saved) {
    // the caller's log-sum-exp, in the rows' log2 units and padded layout
    p3.lsej = ba::LseJob{lse_saved, lse, B * H, static_cast<int>(N), static_cast<int>(BL.fwd.Npad)};
    p3.lse_blocks = (B * H * BL.fwd.Npad + ba::kThreads - 1) / ba::kThreads;
  }
  // delta_i = <dO_i, O_i> for both roles, two threads per row
  p3.delta = ba::DeltaJob{saved ? static_cast<const uint16_t*>(o_saved) : obuf, static_cast<const uint16_t*>(dout),
                          delta, B * H, static_cast<int>(N), static_cast<int>(BL.fwd.Npad), d};
  p3.delta_blocks = (2 * B * H * BL.fwd.Npad + ba::kThreads - 1) / ba::kThreads;
  // 6. the table gradient: the sum of the query role's per-workgroup shares
  ba::PrologueArgs p6{};
  if (dtable) {
    p6.dtr = ba::DtReduceJob{reinterpret_cast<const float*>(ws + BL.dtpart), dtable, static_cast<int>(B),
                             static_cast<int>(H), fp.f.nqt, gh, gw, BL.prow, mode == ba::kBiasRows ? 1 : 0};
    p6.dtr_blocks = (tcount + ba::kDtEntries - 1) / ba::kDtEntries;
  }
  // 4. query role: dq (and the table gradient's shares)
  ba::BwdArgs bq{};
  bq.f = fp.f;
  bq.xrow = static_cast<const uint16_t*>(dout);
  bq.ynat = static_cast<const uint16_t*>(v);
  bq.zt = reinterpret_cast<const uint16_t*>(ws + BL.kst);
  bq.lse = lse;
  bq.delta = delta;
  bq.out1 = dq;
  bq.dtable = dtable;
  bq.dtpart = reinterpret_cast<float*>(ws + BL.dtpart);
  bq.vmax = vmax;
  bq.prow = BL.prow;
  bq.scale = scale;
  // 5. key role: dk, dv; queries and keys exchanged, the bias flipped
  ba::BwdArgs bk = bq;
  bk.f.q = static_cast<const uint16_t*>(k);
  bk.f.kop = reinterpret_cast<const uint32_t*>(ws + BL.qop);
  bk.f.alpha_k = reinterpret_cast<const float*>(ws + BL.alpha_q);
  bk.f.kmax_blk = reinterpret_cast<const float*>(ws + BL.qmax);
  if (mode == ba::kBiasRows) {
    bk.f.bias4 = reinterpret_cast<const float*>(ws + BL.bias4f);
    bk.f.bias_row_max = reinterpret_cast<const float*>(ws + BL.rowmaxf);
  }
  bk.f.table_flip = 1;
  bk.xrow = static_cast<const uint16_t*>(v);
  bk.ynat = static_cast<const uint16_t*>(dout);
  bk.zt = reinterpret_cast<const uint16_t*>(ws + BL.dot);
  bk.zt2 = reinterpret_cast<const uint16_t*>(ws + BL.qst);
  bk.out1 = dk;
  bk.out2 = dv;
  bk.dtable = nullptr;
  for (int role = 0; role < 2; ++role) {
    ba::BwdArgs& b = role == 0 ? bq : bk;
    const int sl = ba::bwd_static_lds(role, b.f.dpad, mode);
    // the query role keeps a table-sized gradient accumulator after the table
    const int tl = ba::fwd_table_lds(b.f, mode) * ((role == 0 && dtable) ? 2 : 1);
    if (sl + tl > kMaxLds) return fail(BA_ERR_UNSUPPORTED, "the backward's tiles and bias table do not fit in LDS");
    b.f.dyn_lds = tl;
    b.f.prio_balance = 0;
  }

  int err = ba::launch_prologue(p1, stream);
  if (err == 0 && !saved) err = ba::launch_attention(f, mode, stream);
  if (err == 0) err = ba::launch_prologue(p3, stream);
  if (err != 0) return hip_fail(err, "backward launch");
  // After the second prologue the two roles depend on nothing of each other
  // (they share inputs only; dtable is checked apart from dk and dv): with
  // the table gradient and N >= 1024 the key role runs on the side stream
  // beside the query role and the table-gradient reduction.  The query role
  // then carries the extra table-gradient work, and each role alone fits two
  // workgroups per CU, leaving its grid's last wave on part of the CUs, which
  // the other role's workgroups fill (detection shape with the table rows:
  // 651 -> 611 us).  Without the table gradient it gains nothing, and on
  // short sequences the fork and join cost more than they save (ViT-Base
  // 14x14: 141 -> 152 us).
  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  SideStream* ss = nullptr;
  if (dtable && N >= 1024) {
    lock.lock();
    ss = side_stream_for(stream);
  }
  hipStream_t main_s = static_cast<hipStream_t>(stream);
  if (ss) {
    err = static_cast<int>(hipEventRecord(ss->fork, main_s));
    if (err == 0) err = static_cast<int>(hipStreamWaitEvent(ss->s, ss->fork, 0));
    if (err != 0) return hip_fail(err, "backward fork");  // nothing is queued on the side stream yet
  }
  if (err == 0) err = ba::launch_backward(bk, ba::kRoleKV, mode, ss ? static_cast<void*>(ss->s) : stream);
  if (err == 0) err = ba::launch_backward(bq, ba::kRoleQ, mode, stream);
  if (err == 0 && dtable) err = ba::launch_prologue(p6, stream);
  if (ss) {
    // Once forked, the caller's stream always waits for the side stream,
    // also when a launch above failed: the key role may be running on the
    // caller's buffers and the workspace.  If the join itself cannot be
    // queued, the host waits for the side stream instead.
    int jerr = static_cast<int>(hipEventRecord(ss->join, ss->s));
    if (jerr == 0) jerr = static_cast<int>(hipStreamWaitEvent(main_s, ss->join, 0));
    if (jerr != 0) (void)hipStreamSynchronize(ss->s);
    if (err == 0) err = jerr;
  }
  if (err != 0) return hip_fail(err, "backward launch");
  return BA_OK;
}

}  // namespace

extern "C" {

ba_status ba_attention_bwd(const void* q, const void* k, const void* v, const void* bias, int gh, int gw,
                           int64_t B, int64_t H, int64_t N, int d, float scale, const void* dout, float* dq,
                           float* dk, float* dv, float* dtable, void* workspace, size_t ws_bytes, void* stream) {
  return run_backward(q, k, v, bias, gh, gw, B, H, N, d, scale, nullptr, nullptr, dout, dq, dk, dv, dtable,
                      workspace, ws_bytes, stream);
}

ba_status ba_attention_bwd_saved(const void* q, const void* k, const void* v, const void* bias, int gh, int gw,
                                 int64_t B, int64_t H, int64_t N, int d, float scale, const void* o,
                                 const float* lse, const void* dout, float* dq, float* dk, float* dv,
                                 float* dtable, void* workspace, size_t ws_bytes, void* stream) {
  if (!o || !lse) return fail(BA_ERR_NULL, "o and lse must be non-NULL");
  return run_backward(q, k, v, bias, gh, gw, B, H, N, d, scale, o, lse, dout, dq, dk, dv, dtable, workspace,
                      ws_bytes, stream);
}

size_t ba_workspace_bytes_bwd(int64_t B, int64_t H, int64_t N, int d, int gh, int gw) {
  if (check_dims(B, H, N, d) != BA_OK || (d != 32 && d != 64 && d != 128)) return 0;
  const bool has_bias = gh > 0 || gw > 0;
  if (has_bias && (gh < 1 || gw < 1 || static_cast<int64_t>(gh) * gw != N)) return 0;
  const BwdLayout L = bwd_layout(B, H, N, d, has_bias, gh, gw);
  if (L.fwd.mode < 0 || L.fwd.mode == kModeExpand) return 0;
  return static_cast<size_t>(L.total);
}

ba_status ba_qk_int_dot(const uint32_t* qbits, const uint32_t* kbits, int64_t B, int64_t H, int64_t N,
                        int d, int route, int32_t* dots, void* stream) {
  if (!qbits || !kbits || !dots) return fail(BA_ERR_NULL, "qbits, kbits and dots must be non-NULL");
  ba_status st = check_dims(B, H, N, d);
  if (st != BA_OK) return st;
  const bool rowsum = (route & BA_QK_ROWSUM) != 0;
  const int r = route & ~BA_QK_ROWSUM;
  if (r != BA_ROUTE_MFMA_FP4 && r != BA_ROUTE_VALU_POPCOUNT && r != BA_ROUTE_MFMA_INT8)
    return fail(BA_ERR_UNSUPPORTED, "unknown route %d", route);
  if (N > 65535 || B * H > 65535) return fail(BA_ERR_SHAPE, "qk_int_dot needs N <= 65535 and B*H <= 65535");
  if (!rowsum && B * H * N > (int64_t{1} << 40) / N) return fail(BA_ERR_SHAPE, "B*H*N*N exceeds 2^40");
  if (!aligned16(qbits) || !aligned16(kbits) || !aligned16(dots))
    return fail(BA_ERR_ALIGN, "qbits, kbits and dots must be 16-byte aligned");
  ba::DotArgs a{qbits, kbits, dots, B * H, static_cast<int>(N), d, (d + 31) / 32, rowsum ? 1 : 0};
  const int err = ba::launch_qk_dot(a, r, stream);
  if (err != 0) return hip_fail(err, "qk_int_dot launch");
  return BA_OK;
}

}  // extern "C"

// ---- the forward that allocates nothing ------------------------------------
// ba_attention_fwd_static runs ba_attention_fwd on a workspace the library
// keeps in device memory of its own: this array, one copy per device, which
// the runtime places when it loads the library's code on that device and
// keeps until the process ends.  Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, looked up once per device on the
// first call there.

namespace {
constexpr size_t kStaticScratchBytes = size_t{BA_STATIC_SCRATCH_MIB} << 20;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The device address of `scratch` on the current device.
ba_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(BA_ERR_HIP, "no current HIP device (or more than 64 devices)");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(static_cast<int>(e), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(BA_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BA_OK;
}

}  // namespace

extern "C" {

ba_status ba_attention_fwd_static(const void* q, const void* k, const void* v, const void* bias, int gh, int gw,
                                  int64_t B, int64_t H, int64_t N, int d, float scale, void* o, void* stream) {
  ba_status st = check_dims(B, H, N, d);
  if (st != BA_OK) return st;
  const bool has_bias = bias != nullptr;
  if (has_bias && (gh < 1 || gw < 1 || static_cast<int64_t>(gh) * gw != N))
    return fail(BA_ERR_SHAPE, "with a bias table gh*gw must equal N (gh=%d gw=%d N=%lld)", gh, gw, (long long)N);
  const Layout L = layout(B, H, N, d, has_bias, has_bias ? gh : 0, has_bias ? gw : 0, false, true);
  if (L.mode < 0)
    return fail(BA_ERR_UNSUPPORTED, "bias grid %dx%d: the table rows do not fit the tile window and the table "
                "exceeds 48 KiB", gh, gw);
  if (static_cast<size_t>(L.total) > kStaticScratchBytes)
    return fail(BA_ERR_WORKSPACE, "the problem needs %lld bytes of scratch; ba_attention_fwd_static keeps %zu "
                "(use ba_attention_fwd with a workspace)", (long long)L.total, kStaticScratchBytes);
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != BA_OK) return st;
  return run_forward(q, k, v, bias, has_bias ? gh : 0, has_bias ? gw : 0, B, H, N, d, scale, o, nullptr, nullptr,
                     ws, kStaticScratchBytes, stream, nullptr, true);
}

}  // extern "C"
