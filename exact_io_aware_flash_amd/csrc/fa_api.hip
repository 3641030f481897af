// fa_api.hip -- the C ABI: argument validation, dispatch and launch (see include/fa.h).
//
// Every argument is checked before anything is enqueued; an invalid call returns its
// status and launches nothing. There is no alternative code path: a combination this
// library does not implement is reported as FA_ERR_UNSUPPORTED, never computed some
// other way (blog "Apakah Konteks Sehari Penuh Mengalahkan Konteks Sepuluh Menit?",
// section "Integrasinya delapan baris": a silent fallback to the slow path looks
// exactly like a slow working model).
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

using namespace fa;

// Scratch of the allocation-free backward (fa_bwd_noalloc): a fixed device array of the
// library, one per GPU, holding what fa_bwd keeps in the caller's workspace. Host code
// never uses the name below as an address (on the host it is only a stand-in for the
// symbol); it uses the device address from hipGetSymbolAddress, taken once per device
// on the first call there, with that device current.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The bits of an enum argument as an int. The C caller may pass any int where the header
// says fa_dtype, fa_status or fa_fp8_layout; in C++ using such an enum object with a value
// outside its enumerators' range is undefined, so arguments are validated on these
// copies and used as enums only once valid.
template <typename E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

fa_status check_common(int B, int H, int N_q, int N_k, int d, float scale, int dtype) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || H < 1 || N_q < 1 || N_k < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  // 32-bit indexing inside one (b, h) and for the grid
  if ((long long)N_q * d > INT_MAX || (long long)N_k * d > INT_MAX) return FA_ERR_SHAPE;
  if ((long long)B * H * ((N_q + 63) / 64 + 1) > INT_MAX) return FA_ERR_SHAPE;
  if ((long long)B * H * N_q > INT_MAX) return FA_ERR_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_ARG;
  return FA_OK;
}

// Fills the bias/mask part of an argument block; returns the status.
template <class Args>
fa_status read_desc(const fa_mask_bias_desc* mb, int H, int N_q, int N_k, fa_dtype dtype,
                    int& bias, Args& a) {
  bias = kBiasNone;
  a.key_start = nullptr;
  a.key_end = nullptr;
  a.n_slopes = 1;
  for (int i = 0; i < FA_MAX_SLOPES; ++i) a.slope2[i] = 0.f;
  a.bmask = nullptr;
  a.bq = a.bk = 64;
  a.nkb = 0;
  a.bm_sb = a.bm_sh = 0;
  a.tbias = nullptr;
  a.tb_sb = a.tb_sh = a.tb_si = 0;
  if (mb == nullptr) return FA_OK;
  if (mb->block_mask != nullptr) {
    if (mb->block_q < 64 || mb->block_q % 64 != 0 || mb->block_k < 64 || mb->block_k % 64 != 0)
      return FA_ERR_MASK;
    if (mb->mask_stride_b < 0 || mb->mask_stride_h < 0) return FA_ERR_MASK;
    if (N_q > FA_MAX_SPARSE_N || N_k > FA_MAX_SPARSE_N) return FA_ERR_UNSUPPORTED;
    a.bmask = mb->block_mask;
    a.bq = mb->block_q;
    a.bk = mb->block_k;
    a.nkb = (N_k + mb->block_k - 1) / mb->block_k;
    a.bm_sb = mb->mask_stride_b;
    a.bm_sh = mb->mask_stride_h;
  }
  if (mb->bias_kind != FA_BIAS_NONE && mb->bias_kind != FA_BIAS_DIST_LINEAR &&
      mb->bias_kind != FA_BIAS_TENSOR)
    return FA_ERR_MASK;
  if ((mb->key_start == nullptr) != (mb->key_end == nullptr)) return FA_ERR_MASK;
  if (mb->key_start != nullptr) {
    if (!aligned16(mb->key_start) || !aligned16(mb->key_end)) return FA_ERR_ALIGN;
    a.key_start = mb->key_start;
    a.key_end = mb->key_end;
  }
  if (mb->bias_kind == FA_BIAS_DIST_LINEAR) {
    if (mb->slopes == nullptr) return FA_ERR_NULL;
    if (mb->n_slopes != 1 && mb->n_slopes != H) return FA_ERR_MASK;
    if (mb->n_slopes > FA_MAX_SLOPES) return FA_ERR_UNSUPPORTED;
    for (int i = 0; i < mb->n_slopes; ++i) {
      if (!std::isfinite(mb->slopes[i])) return FA_ERR_ARG;
      a.slope2[i] = mb->slopes[i] * 1.4426950408889634f;
    }
    a.n_slopes = mb->n_slopes;
    bias = kBiasSlope;
  }
  if (mb->bias_kind == FA_BIAS_TENSOR) {
    if (mb->bias == nullptr) return FA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(mb->bias) & 3u) return FA_ERR_ALIGN;
    if (mb->bias_stride_b < 0 || mb->bias_stride_h < 0 || mb->bias_stride_i < 0) return FA_ERR_MASK;
    // a bias tile (up to 64 rows) is addressed by 32-bit byte offsets from its first row
    if (mb->bias_stride_i * 64 + N_k >= (1LL << 30)) return FA_ERR_UNSUPPORTED;
    a.tbias = mb->bias;
    a.tb_sb = mb->bias_stride_b;
    a.tb_sh = mb->bias_stride_h;
    a.tb_si = mb->bias_stride_i;
    bias = kBiasTensor;
  }
  return FA_OK;
}

// Effective key-range count of the split forward and the keys per range (whole tiles).
// n_split == 0: about two (b, h, query block, range) units per compute unit (256 CUs; two
// small-query workgroups fit on one), each range keeping at least four 64-key tiles.
// Measured on decode-like shapes, 512 units beat both fewer and more.
int split_plan(int B, int H, int N_q, int N_k, int d, int n_split, int& split_keys) {
  const long long tiles = (N_k + kFwdTileKeys - 1) / kFwdTileKeys;
  long long n;
  if (n_split == 0) {
    const int rows = fwd16_rows_per_block(d, N_q);
    const long long units = (long long)B * H * ((N_q + rows - 1) / rows);
    const long long want = 512;
    n = std::min(std::max((want + units - 1) / units, 1LL), std::max(tiles / 4, 1LL));
  } else {
    n = std::min<long long>(n_split, tiles);
  }
  const long long per = (tiles + n - 1) / n;
  split_keys = (int)(per * kFwdTileKeys);
  return (int)((N_k + split_keys - 1) / split_keys);
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device id, or NULL

// The current device's scratch address (looked up on first use); NULL on a HIP error.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

size_t split_part_bytes(int B, int H, int N_q, int d, int n) {
  return round256((size_t)n * B * H * N_q * d * sizeof(float));
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (raw(s)) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (B, H, N_q, N_k must be >= 1 and fit 32-bit indexing)";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_HEADDIM: return "head dimension must be 64 or 128";
    case FA_ERR_MASK: return "malformed mask/bias descriptor";
    case FA_ERR_ALIGN: return "device pointer misaligned (16 bytes; 4 for float32 arrays)";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_UNSUPPORTED: return "combination not implemented";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_ARG: return "invalid scalar argument (scale must be finite and > 0)";
    case FA_ERR_SCRATCH:
      return "problem too large for the fixed scratch of fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

const char* fa_version(void) { return "fa 0.1.0 gfx950"; }

int fa_fp8_rows(int N) { return N < 1 ? 0 : ((N + 63) / 64) * 64; }

fa_status fa_fp8_quantize(const void* x, int B, int H, int N, int d, fa_dtype dtype,
                          fa_fp8_layout layout, const float* signs, void* x8, float* amax,
                          void* stream) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (raw(dtype) != FA_BF16 && raw(dtype) != FA_F16) return FA_ERR_DTYPE;
  if (raw(layout) != FA_FP8_Q && raw(layout) != FA_FP8_K && raw(layout) != FA_FP8_V) return FA_ERR_ARG;
  if (!x || !x8 || !amax) return FA_ERR_NULL;
  if (!aligned16(x) || !aligned16(x8) || (reinterpret_cast<uintptr_t>(amax) & 3u)) return FA_ERR_ALIGN;
  if ((long long)N * d > INT_MAX) return FA_ERR_SHAPE;
  const long long np = fa_fp8_rows(N);
  if ((long long)B * H * (np / 64) > INT_MAX) return FA_ERR_SHAPE;  // one workgroup per block
  Fp8QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  if (signs != nullptr) {
    if (layout == FA_FP8_V) return FA_ERR_ARG;
    for (int e = 0; e < d; ++e) {
      if (signs[e] == -1.f) a.sign_bits[e >> 5] |= 1u << (e & 31);
      else if (signs[e] != 1.f) return FA_ERR_ARG;
    }
    a.rotate = 1;
  }
  a.x = x; a.x8 = static_cast<uint8_t*>(x8); a.amax = amax;
  a.B = B; a.H = H; a.N = N; a.Np = (int)np;
  a.layout = layout;
  const hipError_t e = launch_fp8_quant(dtype, d, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_amax,
                     const float* k_amax, const float* v_amax, void* o, float* lse, int B, int H,
                     int N_q, int N_k, int d, float scale, int causal, int rotated,
                     fa_dtype out_dtype, void* stream) {
  fa_status st = check_common(B, H, N_q, N_k, d, scale, FA_BF16);
  if (st != FA_OK) return st;
  if (raw(out_dtype) != FA_BF16 && raw(out_dtype) != FA_F16) return FA_ERR_DTYPE;
  if (!q8 || !k8 || !v8 || !q_amax || !k_amax || !v_amax || !o) return FA_ERR_NULL;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o)) return FA_ERR_ALIGN;
  if (((reinterpret_cast<uintptr_t>(q_amax) | reinterpret_cast<uintptr_t>(k_amax) |
        reinterpret_cast<uintptr_t>(v_amax)) & 3u) ||
      (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return FA_ERR_ALIGN;
  Fp8FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q8 = static_cast<const uint8_t*>(q8);
  a.k8 = static_cast<const uint8_t*>(k8);
  a.v8 = static_cast<const uint8_t*>(v8);
  a.q_amax = q_amax; a.k_amax = k_amax; a.v_amax = v_amax;
  a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Nq = N_q; a.Nk = N_k;
  a.Nqp = fa_fp8_rows(N_q); a.Nkp = fa_fp8_rows(N_k);
  a.causal = causal ? 1 : 0;
  a.sl2 = scale * 1.4426950408889634f / (rotated ? (float)d : 1.f);
  const hipError_t e = launch_fwd8(out_dtype, d, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N_q, int N_k, int d, float scale, int causal, const fa_mask_bias_desc* mb,
                 fa_dtype dtype, void* stream) {
  fa_status st = check_common(B, H, N_q, N_k, d, scale, raw(dtype));
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_ALIGN;
  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  int bias = kBiasNone;
  st = read_desc(mb, H, N_q, N_k, dtype, bias, a);
  if (st != FA_OK) return st;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Nq = N_q; a.Nk = N_k;
  a.causal = causal ? 1 : 0;
  a.sl2 = scale * 1.4426950408889634f;
  hipError_t e = launch_fwd(dtype, d, bias, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_tile_counts(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int N_q, int N_k, int d, float scale, int causal,
                             const fa_mask_bias_desc* mb, fa_dtype dtype, void* stream,
                             unsigned long long* counts, int* config) {
  fa_status st = check_common(B, H, N_q, N_k, d, scale, raw(dtype));
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !counts || !config) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(counts) & 7u) return FA_ERR_ALIGN;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;  // counted in the 16-bit kernels only
  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  int bias = kBiasNone;
  st = read_desc(mb, H, N_q, N_k, dtype, bias, a);
  if (st != FA_OK) return st;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Nq = N_q; a.Nk = N_k;
  a.causal = causal ? 1 : 0;
  a.sl2 = scale * 1.4426950408889634f;
  a.counts = counts;
  hipError_t e = launch_fwd(dtype, d, bias, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return FA_ERR_HIP;
  config[0] = a.rows_wg;
  config[1] = 32;  // query rows per wave
  config[2] = a.keys_tile;
  return FA_OK;
}

int fa_fwd_split_count(int B, int H, int N_q, int N_k, int d, int n_split) {
  if (n_split < 0 || check_common(B, H, N_q, N_k, d, 1.f, FA_BF16) != FA_OK) return 0;
  int sk = 0;
  return split_plan(B, H, N_q, N_k, d, n_split, sk);
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int N_q, int N_k, int d, int n_split) {
  const int n = fa_fwd_split_count(B, H, N_q, N_k, d, n_split);
  if (n <= 1) return 0;
  return split_part_bytes(B, H, N_q, d, n) + round256((size_t)n * B * H * N_q * sizeof(float));
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N_q, int N_k, int d, float scale, int causal,
                       const fa_mask_bias_desc* mb, fa_dtype dtype, int n_split, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (n_split < 0) return FA_ERR_ARG;
  fa_status st = check_common(B, H, N_q, N_k, d, scale, raw(dtype));
  if (st != FA_OK) return st;
  int split_keys = 0;
  const int n = split_plan(B, H, N_q, N_k, d, n_split, split_keys);
  if (n <= 1)
    return fa_fwd(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, mb, dtype, stream);
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_ALIGN;
  if (workspace == nullptr ||
      workspace_bytes < fa_fwd_split_workspace_bytes(B, H, N_q, N_k, d, n_split))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  int bias = kBiasNone;
  st = read_desc(mb, H, N_q, N_k, dtype, bias, a);
  if (st != FA_OK) return st;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Nq = N_q; a.Nk = N_k;
  a.causal = causal ? 1 : 0;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_split = n;
  a.split_keys = split_keys;
  a.o_part = static_cast<float*>(workspace);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        split_part_bytes(B, H, N_q, d, n));
  hipError_t e = launch_fwd(dtype, d, bias, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N_q, int N_k, int d) {
  (void)d;
  if (B < 1 || H < 1 || N_q < 1 || N_k < 1) return 0;
  // delta = rowsum(dO * O) (one float per query row) + the key-range summary of every
  // 64-row query tile (4 int32) + LSE * log2(e) (one float per query row) + one float
  // per (b, h, 128-key block) for the slope gradient, each rounded up to 256 bytes
  return bwd_workspace_bytes(B, H, N_q, N_k);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, fa_dtype grad_dtype,
                 void* workspace, size_t workspace_bytes, int B, int H, int N_q, int N_k, int d,
                 float scale, int causal, const fa_mask_bias_desc* mb, fa_dtype dtype,
                 void* stream) {
  return fa_bwd_phases(FA_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, grad_dtype, workspace,
                       workspace_bytes, B, H, N_q, N_k, d, scale, causal, mb, dtype, stream);
}

}  // extern "C"

namespace {

// Validation of a backward call, everything except the workspace (shared by fa_bwd_phases
// and fa_bwd_noalloc); fills the argument block's descriptor part.
fa_status bwd_check(int phases, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    fa_dtype grad_dtype, int B, int H, int N_q, int N_k, int d, float scale,
                    const fa_mask_bias_desc* mb, fa_dtype dtype, int& bias, BwdArgs& a) {
  if (phases < 1 || (phases & ~(FA_BWD_ALL | FA_BWD_DQ_ATOMIC)) != 0) return FA_ERR_ARG;
  const bool dqa = (phases & FA_BWD_DQ_ATOMIC) != 0;
  if (dqa && ((phases & FA_BWD_DKDV) == 0 || (phases & FA_BWD_DQ) != 0)) return FA_ERR_ARG;
  fa_status st = check_common(B, H, N_q, N_k, d, scale, raw(dtype));
  if (st != FA_OK) return st;
  if (raw(grad_dtype) != FA_F32 && raw(grad_dtype) != raw(dtype)) return FA_ERR_DTYPE;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  const void* dev[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : dev)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return FA_ERR_ALIGN;
  std::memset(&a, 0, sizeof(a));
  bias = kBiasNone;
  st = read_desc(mb, H, N_q, N_k, dtype, bias, a);
  if (st != FA_OK) return st;
  if (mb != nullptr && mb->dslopes != nullptr) {
    if (mb->bias_kind != FA_BIAS_DIST_LINEAR) return FA_ERR_MASK;
    if (reinterpret_cast<uintptr_t>(mb->dslopes) & 3u) return FA_ERR_ALIGN;
  }
  if (mb != nullptr && mb->dbias != nullptr) {
    if (mb->bias_kind != FA_BIAS_TENSOR) return FA_ERR_MASK;
    if (reinterpret_cast<uintptr_t>(mb->dbias) & 3u) return FA_ERR_ALIGN;
  }
  if (mb != nullptr && mb->dbias_reduce != 0) {
    const int all = FA_DBIAS_SUM_BATCH | FA_DBIAS_SUM_HEADS | FA_DBIAS_SUM_ROWS;
    if (mb->dbias == nullptr || (mb->dbias_reduce & ~all) != 0) return FA_ERR_MASK;
  }
  if (dqa && (raw(grad_dtype) != FA_F32 || raw(dtype) == FA_F32 || a.bmask != nullptr ||
              bias == kBiasTensor))
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Launches of a validated backward call with `workspace` (fa_bwd_workspace_bytes bytes).
fa_status bwd_launch(int phases, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     fa_dtype grad_dtype, void* workspace, int B, int H, int N_q, int N_k, int d,
                     float scale, int causal, const fa_mask_bias_desc* mb, fa_dtype dtype,
                     int bias, BwdArgs& a, void* stream) {
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.qsum = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + bwd_qsum_offset(B, H, N_q));
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_lse2_offset(B, H, N_q));
  if (mb != nullptr && mb->dslopes != nullptr) {
    a.dslopes = mb->dslopes;
    a.dslope_part =
        reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_dslope_offset(B, H, N_q));
  }
  if (mb != nullptr && mb->dbias != nullptr) {
    a.dbias = mb->dbias;
    a.db_red = mb->dbias_reduce;
  }
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = B; a.H = H; a.Nq = N_q; a.Nk = N_k;
  a.causal = causal ? 1 : 0;
  a.grad_f32 = grad_dtype == FA_F32 ? 1 : 0;
  a.scale = scale;
  a.sl2 = scale * 1.4426950408889634f;
  hipError_t e = launch_bwd(dtype, d, bias, phases, a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return FA_ERR_UNSUPPORTED;
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_bwd_phases(int phases, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        fa_dtype grad_dtype, void* workspace, size_t workspace_bytes, int B,
                        int H, int N_q, int N_k, int d, float scale, int causal,
                        const fa_mask_bias_desc* mb, fa_dtype dtype, void* stream) {
  BwdArgs a;
  int bias = kBiasNone;
  fa_status st = bwd_check(phases, q, k, v, o, lse, dout, dq, dk, dv, grad_dtype, B, H, N_q, N_k,
                           d, scale, mb, dtype, bias, a);
  if (st != FA_OK) return st;
  if (workspace == nullptr || workspace_bytes < fa_bwd_workspace_bytes(B, H, N_q, N_k, d))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  return bwd_launch(phases, q, k, v, o, lse, dout, dq, dk, dv, grad_dtype, workspace, B, H, N_q,
                    N_k, d, scale, causal, mb, dtype, bias, a, stream);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         fa_dtype grad_dtype, int B, int H, int N_q, int N_k, int d, float scale,
                         int causal, const fa_mask_bias_desc* mb, fa_dtype dtype, void* stream) {
  BwdArgs a;
  int bias = kBiasNone;
  fa_status st = bwd_check(FA_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, grad_dtype, B, H, N_q,
                           N_k, d, scale, mb, dtype, bias, a);
  if (st != FA_OK) return st;
  if (fa_bwd_workspace_bytes(B, H, N_q, N_k, d) > (size_t)FA_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_SCRATCH;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return FA_ERR_HIP;
  // Everything the launches read from the scratch is written earlier in the same call
  // (prep: D and the exponent offsets; key-range summary; every dK/dV workgroup writes
  // its slope-gradient partial), so the previous call's contents need no clearing.
  return bwd_launch(FA_BWD_ALL, q, k, v, o, lse, dout, dq, dk, dv, grad_dtype, ws, B, H, N_q,
                    N_k, d, scale, causal, mb, dtype, bias, a, stream);
}

fa_status fa_mask_summary(const int32_t* key_start, const int32_t* key_end, int N_q, int N_k,
                          int block_rows, int32_t* out, void* stream) {
  if (!key_start || !key_end || !out) return FA_ERR_NULL;
  if (N_q < 1 || N_k < 1) return FA_ERR_SHAPE;
  if (block_rows < 1 || block_rows > 1024) return FA_ERR_SHAPE;
  if (!aligned16(key_start) || !aligned16(key_end) || !aligned16(out)) return FA_ERR_ALIGN;
  hipError_t e = launch_mask_summary(key_start, key_end, N_q, N_k, block_rows, out,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
