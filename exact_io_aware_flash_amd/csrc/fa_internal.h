// fa_internal.h -- host/device argument blocks and launcher declarations (library-private).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// Work-to-workgroup mapping of the forward/backward grids.
enum Sched : int {
  kSchedHeadMajor = 0,  // block L -> head L / nblk, heaviest query block first
  kSchedXcd = 1,        // heads pinned to one of the 8 XCDs (L % 8), heaviest first
  kSchedXcdLpt = 2      // as kSchedXcd, blocks of all the XCD's heads by weight
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* key_start;  // NULL: no key-range mask
  const int32_t* key_end;
  int B, H, Nq, Nk;
  int causal;
  int nqb;     // query blocks per (b, h)
  int sched;   // Sched
  int n_slopes;
  float sl2;   // scale * log2(e)
  float slope2[FA_MAX_SLOPES];  // bias slope * log2(e), per head or broadcast
  // split-key forward (n_split > 1): keys [r * split_keys, (r+1) * split_keys) per range r
  int n_split;
  int split_keys;   // multiple of the 64-key tile
  float* o_part;    // [n_split][B*H*Nq][d] float32 normalised partial outputs
  float* lse_part;  // [n_split][B*H*Nq] float32 partial LSE (-inf: nothing visible)
  // block-sparse bitmap (NULL: none): byte (r, c) of head (b, h) at
  // bmask[b * bm_sb + h * bm_sh + r * nkb + c] for blocks of bq rows x bk keys
  const uint8_t* bmask;
  int bq, bk, nkb;
  long long bm_sb, bm_sh;
  // float32 bias tensor (bias mode 2): element (b, h, i, j) at
  // tbias[b * tb_sb + h * tb_sh + i * tb_si + j]
  const float* tbias;
  long long tb_sb, tb_sh, tb_si;
  // tile counters (NULL: off): [0] += key tiles each workgroup loads, [1] += (wave, tile)
  // score blocks computed; the 16-bit launcher reports its workgroup rows and tile keys
  unsigned long long* counts;
  int rows_wg, keys_tile;
};

// The split-key 16-bit forward uses a smaller workgroup (4 waves, 32-key tiles, 64 KB of
// LDS, so two workgroups share a compute unit) when a head has at most this many rows.
constexpr int kFwdFewRows = 64;
// Nominal query rows per work unit of the 16-bit forward, used to plan the automatic
// split count (for N_q <= kFwdFewRows a head is one query block in every configuration;
// for d = 128 and more rows the launch picks 256- or 128-row workgroups by grid size).
inline int fwd16_rows_per_block(int d, int Nq) { return (d == 128 && Nq > kFwdFewRows) ? 256 : 128; }
// Split ranges are multiples of this many keys (a multiple of every forward tile).
constexpr int kFwdTileKeys = 64;

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;   // [B,H,Nq] rowsum(dO * O), workspace (negated by the 16-bit prep pass)
  float* lse2;    // [B,H,Nq] LSE * log2(e), workspace
  int32_t* qsum;  // key-range summary per query tile of the dK/dV pass, workspace
  void* dq;
  void* dk;
  void* dv;
  const int32_t* key_start;
  const int32_t* key_end;
  int B, H, Nq, Nk;
  int causal;
  int nblk;      // blocks per (b, h) along the parallel axis of the kernel
  int sched;
  int grad_f32;  // 1: gradients written as float32, else in the input type
  int n_slopes;
  float scale;
  float sl2;
  float slope2[FA_MAX_SLOPES];
  // slope gradient (NULL: not wanted): per-workgroup partial sums of dS |i - j| of the
  // dK/dV pass [B*H][nblk] in the workspace, reduced into dslopes[n_slopes]
  float* dslope_part;
  float* dslopes;
  // block-sparse bitmap, as in FwdArgs
  const uint8_t* bmask;
  int bq, bk, nkb;
  long long bm_sb, bm_sh;
  // bias tensor, as in FwdArgs; dbias (NULL: not wanted) dense [B',H',Nq',Nk] float32,
  // summed over the axes of db_red (FA_DBIAS_SUM_* bits)
  const float* tbias;
  long long tb_sb, tb_sh, tb_si;
  float* dbias;
  int db_red;
};

// Bias modes of the kernels: none, slope * |i - j| generated on the fly, float32 tensor.
enum BiasMode : int { kBiasNone = 0, kBiasSlope = 1, kBiasTensor = 2 };

// Launchers (return hipSuccess or the launch error). dtype-specialised in the .hip files.
hipError_t launch_fwd(fa_dtype dt, int d, int bias_mode, FwdArgs& a, hipStream_t st);
// Tiles of the block-sparse forward list per workgroup (keys per tile >= 32).
constexpr int kSparseMaxTiles = FA_MAX_SPARSE_N / 32;
hipError_t launch_bwd(fa_dtype dt, int d, int bias_mode, int phases, BwdArgs& a, hipStream_t st);
// float32 inputs (fa_bwd32.hip): prep, dK/dV and dQ passes on float32 MFMA
hipError_t launch_bwd32(int d, int bias_mode, int phases, BwdArgs& a, hipStream_t st);
// dL/dslope from the dK/dV pass's per-workgroup partials [B*H][nblk], in a fixed order
hipError_t launch_dslope_reduce(const float* part, int B, int H, int nblk, int n_slopes,
                                float* out, hipStream_t st);
// query rows per LDS tile of the 16-bit dK/dV pass: the granularity of the key-range
// summary in the backward workspace
constexpr int kDkdvBR = 64;
hipError_t launch_mask_summary(const int32_t* ks, const int32_t* ke, int Nq, int Nk, int block,
                               int32_t* out, hipStream_t st);

// Backward workspace layout: delta at offset 0, key-range summary at bwd_qsum_offset,
// LSE * log2(e) at bwd_lse2_offset.
size_t bwd_qsum_offset(int B, int H, int Nq);
size_t bwd_lse2_offset(int B, int H, int Nq);
size_t bwd_dslope_offset(int B, int H, int Nq);
size_t bwd_workspace_bytes(int B, int H, int Nq, int Nk);

// FP8 quantiser (fa_fp8_quantize): one launch per tensor (V: an amax pass first)
struct Fp8QuantArgs {
  const void* x;       // [B,H,N,d] 16-bit input
  uint8_t* x8;         // [B,H,Np,d] E4M3 codes in the layout's byte order
  float* amax;         // [B,H,Np/64] block amax (V: written by the first pass)
  int B, H, N, Np;     // Np = N rounded up to 64
  int layout;          // fa_fp8_layout
  int rotate;          // 1: multiply rows by diag(signs) H_d first (Q, K)
  uint32_t sign_bits[4];  // bit e set: sign of column e is -1
};

// FP8 forward (fa_fwd_fp8)
struct Fp8FwdArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* q_amax;
  const float* k_amax;
  const float* v_amax;
  void* o;
  float* lse;
  int B, H, Nq, Nk, Nqp, Nkp;
  int causal;
  int nqb;
  int sched;
  float sl2;  // scale * log2(e), divided by d for rotated Q and K
};

hipError_t launch_fp8_quant(fa_dtype dt, int d, Fp8QuantArgs& a, hipStream_t st);
hipError_t launch_fwd8(fa_dtype out, int d, Fp8FwdArgs& a, hipStream_t st);

}  // namespace fa
