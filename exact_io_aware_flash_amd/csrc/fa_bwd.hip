// fa_bwd.hip -- recompute-based attention backward for gfx950 (MI355X).
//
// Method (blog "Apakah Konteks Sehari Penuh Mengalahkan Konteks Sepuluh Menit?", section
// "Backward pass: menghitung ulang, bukan menyimpan"): only O and the softmax statistics
// (here the log-sum-exp) are kept from the forward pass; every score tile is recomputed
// from Q and K, P = exp(S - LSE). The gradient formulas are the textbook softmax
// Jacobian: dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
// dQ = scale * dS K, dK = scale * dS^T Q.
//
// Three launches, no atomics, deterministic:
//  1. prep:  D_i = rowsum(dO_i * O_i) in float32 (one HBM pass), stored negated, and
//            LSE_i * log2(e);
//  2. dkdv:  one workgroup per (b, h, block of 32*NW keys); each wave keeps its 32 keys'
//            K and V rows in registers and accumulates dK^T/dV^T while walking the query
//            tiles. S = Q K^T and dP = dO V^T come out with the key on the lane and the
//            query on the register, so P^T and dS^T feed the dV/dK products straight from
//            registers; Q and dO are staged in LDS both row-major (A operands of S, dP)
//            and transposed (B operands of dV, dK);
//  3. dq:    forward-shaped: one workgroup per (b, h, block of 32*NW queries); Q, dO, LSE
//            and D of the wave's 32 queries stay in registers; K (read as rows and by
//            transposing gathers) and V tiles stream through a ring of LDS stages;
//            dQ^T += K^T dS^T.
// The dq pass recomputes S and dP a second time (7 matrix products instead of 5) in
// exchange for no float32 atomics on dQ.
#include <algorithm>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// ---------------------------------------------------------------------------------
// 1. D = rowsum(dO * O)
// ---------------------------------------------------------------------------------
// D is stored negated: the dK/dV pass starts its dP accumulation from it, so the MFMA
// chain delivers dP - D directly. Also writes the exponent offset per row (lse_offset2:
// LSE * log2(e)), which the dK/dV pass reads.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T* __restrict__ o,
                                                       const T* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ delta,
                                                       float* __restrict__ lse2, int rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements (16 bytes) each
  constexpr int RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + (int)threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 x = ldg16(o + (size_t)row * D + c * 8);
    const u32x4 y = ldg16(dout + (size_t)row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t xw = x[w], yw = y[w];
      const float x0 = (float)__builtin_bit_cast(T, (uint16_t)(xw & 0xffffu));
      const float x1 = (float)__builtin_bit_cast(T, (uint16_t)(xw >> 16));
      const float y0 = (float)__builtin_bit_cast(T, (uint16_t)(yw & 0xffffu));
      const float y1 = (float)__builtin_bit_cast(T, (uint16_t)(yw >> 16));
      acc = __builtin_fmaf(x0, y0, acc);
      acc = __builtin_fmaf(x1, y1, acc);
    }
  }
#pragma unroll
  for (int s = TPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && c == 0) {
    delta[row] = -acc;
    lse2[row] = lse_offset2(lse[row]);
  }
}

// Stores 4 consecutive float gradients (converted as requested).
template <typename T>
__device__ inline void store_grad4(void* base, size_t idx, bool f32, float v0, float v1, float v2,
                                   float v3) {
  if (f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = f32x4{v0, v1, v2, v3};
  } else {
    stg8(static_cast<T*>(base) + idx, u32x2{Elt<T>::pack2(v0, v1), Elt<T>::pack2(v2, v3)});
  }
}

// ---------------------------------------------------------------------------------
// 2. dK, dV: key-block-outer
// ---------------------------------------------------------------------------------
// Per stage: Q and dO tiles (BR rows, swizzled, filled by direct loads), then the tile's
// LSE*log2(e), D, key_start and key_end (one 4-byte direct load each, BR == 64 == lanes).
template <int D, int BR>
struct DkdvLds {
  static constexpr int RB = 2 * D;
  static constexpr int QT = 0, DT = BR * RB;
  static constexpr int LSE = 2 * BR * RB, DLT = LSE + BR * 4, KS = DLT + BR * 4, KE = KS + BR * 4;
  static constexpr int STAGE = KE + BR * 4;
};

// Query tiles in the dK/dV ring: two stages (one tile in flight) measured 2-3 % faster
// than three or four on the bf16 causal N = 8192 d = 128 shape (1167-1172 against
// 1191-1199 us): the wave is alone on its SIMD and its tile takes long enough for one
// load ahead to land.
#ifndef FA_DKDV_STAGES
#define FA_DKDV_STAGES 2
#endif

// MEM: dbias summed over batches and/or heads (bias tensor only): the member loop below.
// DQA: the pass also forms dQ = scale dS K for its keys and adds it into the float32 dq
// with atomics (no bias tensor, no bitmap).
template <typename T, int D, int BR, int NW, int WPE, int BM, bool SPARSE, bool MEM = false,
          bool DQA = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dkdv_kernel(const BwdArgs a) {
  using E = Elt<T>;
  using L = DkdvLds<D, BR>;
  using Tile = DmaTile<BR, D, NW>;
  using BT = BiasColTile;
  constexpr bool BIAS = BM == kBiasSlope, TENSOR = BM == kBiasTensor;
  constexpr int BK = 32 * NW, QB = BR / 32, DK = D / 16, DB = D / 32, RB = L::RB;
  constexpr int ST = FA_DKDV_STAGES, P = ST - 1;
  // Q, dO windows + one row array (+ the wave's bias windows)
  constexpr int kOpsPerTile = 2 * Tile::kOpsPerWave + 1 + (TENSOR ? BT::kOps : 0);
  // a stage: Q, dO, row arrays (+ each wave's bias windows)
  constexpr int kStage = L::STAGE + (TENSOR ? NW * BT::kWaveBytes : 0);
  static_assert(BR == 64 && NW == 4, "one row array (64 entries) per wave");
  // with the bias tensor the loop's only wait is the full one (the dbias stores count
  // in the same counter as the direct loads)
  static_assert(!TENSOR || ST == 2, "bias tensor: one tile in flight");
  // dQ by atomics: one tile in flight (its waits are full ones: the atomics count in the
  // same counter as the direct loads)
  static_assert(!DQA || (!TENSOR && !SPARSE && ST == 2), "dQ atomics: plain or slope bias");
  static_assert(P * kOpsPerTile < 64, "vmcnt range");
  static_assert(ST * kStage <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[ST * kStage];
  __shared__ int win[2];
  // dQ by atomics: dS^T of a query tile (BK keys x BR queries, 16-bit, rows of 2 BR bytes
  // swizzled like 64-column tiles), two buffers used by alternate tiles
  constexpr int kDsBuf = BK * BR * 2;
  __shared__ __attribute__((aligned(1024))) char dst_s[DQA ? 2 * kDsBuf : 16];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, n = lane & 31, h = lane >> 5;
  const int wid_s = wave_id();  // the same index as a scalar, for LDS window bases
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const bool causal = a.causal != 0, ranged = a.key_start != nullptr;
  // dbias summed over batches and/or heads: the workgroup owns one dbias slice (slot) and
  // computes, one after the other, every (b, h) that shares it (its members), so each
  // element is summed by one thread in a fixed order; otherwise a slot is one (b, h)
  static_assert(!MEM || TENSOR, "member loop: bias tensor only");
  const int rb = MEM ? (a.db_red & FA_DBIAS_SUM_BATCH) : 0;
  const int rh = MEM ? (a.db_red & FA_DBIAS_SUM_HEADS) : 0;
  const bool rrows = TENSOR && (a.db_red & FA_DBIAS_SUM_ROWS) != 0;
  const int slot_h = rh ? 1 : a.H;                    // heads of the dbias array
  const int n_slots = (rb ? 1 : a.B) * slot_h;
  const int mem_h = rh ? a.H : 1, n_mem = (rb ? a.B : 1) * mem_h;
  int slot, kb;
  map_block(blockIdx.x, n_slots, a.nblk, a.sched, false, slot, kb);
  float* dB = nullptr;  // the slot's dbias [Nq' rows][Nk] (NULL: dbias not wanted)
  if constexpr (TENSOR)
    if (a.dbias != nullptr) dB = a.dbias + (size_t)slot * (rrows ? 1 : Nq) * Nk;
  float dbr = 0.f;  // rows summed: this lane's share of its key's dbias, over all members

  for (int m = 0; m < n_mem; ++m) {
    if (m > 0) __syncthreads();  // every wave is done with the ring and the tile list
    // the first member writes dbias, later ones add to it; with a bitmap a member may skip
    // tiles another one visits, so the launch clears dbias and every member adds
    const bool first = m == 0 && !(SPARSE && MEM);
    const int bh = (rb | rh) ? (rb ? m / mem_h : slot / slot_h) * a.H
                                   + (rh ? m % mem_h : slot % slot_h)
                             : slot;
    const int head = bh % a.H;
    const T* Q = static_cast<const T*>(a.q) + (size_t)bh * Nq * D;
    const T* K = static_cast<const T*>(a.k) + (size_t)bh * Nk * D;
    const T* V = static_cast<const T*>(a.v) + (size_t)bh * Nk * D;
    const T* dO = static_cast<const T*>(a.dout) + (size_t)bh * Nq * D;
    const float sl2 = a.sl2;
    const float slope2 = BIAS ? a.slope2[a.n_slopes == 1 ? 0 : head] : 0.f;
    const float* TB = TENSOR ? a.tbias + (long long)(bh / a.H) * a.tb_sb + (long long)head * a.tb_sh
                             : nullptr;

    const int k0 = kb * BK, k1 = min(k0 + BK, Nk);
    const int kw0 = k0 + 32 * wid, kw1 = min(kw0 + 32, Nk);
    const int key = kw0 + n;  // this lane's key (column of S)

    // K and V rows of the wave's keys: B operands of S = Q K^T and dP = dO V^T
    u32x4 kf[DK], vf[DK];
    {
      const size_t r = (size_t)min(key, Nk - 1);
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        kf[ks] = ldg16(K + r * D + 16 * ks + 8 * h);
        vf[ks] = ldg16(V + r * D + 16 * ks + 8 * h);
      }
    }

    // dQ by atomics: wave w forms the d columns 32 dbw .. 32 dbw + 31 of dQ (both 32-row
    // blocks of a tile for d = 128; block w / 2 for d = 64) over the workgroup's BK keys.
    // kt[s]: its B operands K^T (keys 16s + 8p + 4h + i, i < 4, p < 2, as the transposing
    // reads deliver them), gathered once from the block's K rows staged in ring stage 0,
    // which the prologue below has not yet filled.
    constexpr int NS = DQA ? BK / 16 : 1;
    const int dbw = wid_s % DB;
    const int q4 = (lane >> 2) & 3, g16 = (lane >> 4) & 1, lo2 = lane & 3;
    u32x4 kt[NS];
    if constexpr (DQA) {
      wait_vmem<0>();
      const int rr = 32 * wid + n;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) lds_st16(smem, rr * RB + 16 * ((2 * ks + h) ^ swz<D>(rr)), kf[ks]);
      __syncthreads();
      int o2[2];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int r = 8 * pp + 4 * h + q4;
        o2[pp] = r * RB + 16 * ((4 * dbw + 2 * g16 + (lo2 >> 1)) ^ swz<D>(r)) + 8 * (lo2 & 1);
      }
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const u32x2 lo = lds_ld8_tr(smem, 16 * s2 * RB + o2[0]);
        const u32x2 hi = lds_ld8_tr(smem, 16 * s2 * RB + o2[1]);
        kt[s2] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      __syncthreads();  // every wave holds its fragments before the ring reuses the stage
    }
    char* dsw = dst_s;  // dS^T buffer the current tile writes

    // query tiles that can see a key of this block
    const int nqt = (Nq + BR - 1) / BR;
    int t_lo = 0, t_hi = nqt;
    if (causal) t_lo = max(0, k0 - off) / BR;
    if (causal && k0 - off >= Nq) t_hi = 0;
    if (ranged) {
      if (tid < 64) {
        int lo = nqt, hi = -1;
        for (int t = lane; t < nqt; t += 64) {
          const int* sm = a.qsum + 4 * t;  // {min start, max start, min end, max end}
          if (!(k1 <= sm[0] || k0 >= sm[3])) { lo = min(lo, t); hi = max(hi, t); }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) { win[0] = lo; win[1] = hi + 1; }
      }
      __syncthreads();
      t_lo = max(t_lo, win[0]);
      t_hi = min(t_hi, win[1]);
    }
    if (k0 >= Nk) t_hi = t_lo;

    // block-sparse bitmap: the query tiles the workgroup loads (see build_tile_list); a
    // 64-row query tile and a wave's 32 keys each lie inside one block
    constexpr int kMaxT = SPARSE ? FA_MAX_SPARSE_N / BR : 64;
    __shared__ uint32_t need_w[SPARSE ? NW : 1][2 * (kMaxT / 64)];
    __shared__ uint32_t tlist[SPARSE ? kMaxT : 1];
    __shared__ int n_list_s;
    int n_pos = t_hi - t_lo;
    if constexpr (SPARSE) {
      const uint8_t* bcol = nullptr;
      if (kw0 < Nk) {
        const int bb = bh / a.H, hh = bh - bb * a.H;
        bcol = a.bmask + bb * a.bm_sb + hh * a.bm_sh + kw0 / a.bk;
      }
      n_pos = build_tile_list(need_w, tlist, &n_list_s, wid_s, lane, t_lo, t_hi, [&](int t) {
        const int q0t = t * BR;
        bool skip = bcol == nullptr;
        if (causal) skip |= q0t + BR - 1 + off < kw0;
        if (ranged) {
          const int* sm = a.qsum + 4 * t;
          skip |= kw1 <= sm[0] || kw0 >= sm[3];
        }
        return !skip && bcol[(long long)(q0t / a.bq) * a.nkb] != 0;
      });
    }
    ListWindow<kMaxT> lw;
    if constexpr (SPARSE) lw.init(tlist, lane);
    auto tile_at = [&](int p) -> int {
      if constexpr (SPARSE) return (int)(lw.at(p) & 0xffffu);
      else return t_lo + p;
    };

    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dv[db] = f32x16{}; dk[db] = f32x16{}; }
    float sgrad = 0.f;  // this lane's share of dL/dslope (bias only)

    // LDS offsets inside a swizzled tile (see DmaTile): row reads of query row 32qb + n,
    // chunk 2ks + h (A operands of S and dP); transposing gathers of 8 query rows of one
    // d column (B operands of dV += P^T dO and dK += dS^T Q).
    int ra[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) ra[ks] = n * RB + 16 * ((2 * ks + h) ^ swz<D>(n));
    int ta[DB][2];
    {
      const int q = (lane >> 2) & 3, g16 = (lane >> 4) & 1, lo2 = lane & 3;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int r = 8 * p + 4 * h + q;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          ta[db][p] = r * RB + 16 * ((4 * db + 2 * g16 + (lo2 >> 1)) ^ swz<D>(r)) + 8 * (lo2 & 1);
      }
    }
    auto cfrag = [&](const char* base, int qb, int st, int db) {
      const int rows = (32 * qb + 16 * st) * RB;
      const u32x2 lo = lds_ld8_tr(base, rows + ta[db][0]);
      const u32x2 hi = lds_ld8_tr(base, rows + ta[db][1]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };

    // one 32-query block of a tile; MASK: per-element visibility
    float pre[TENSOR ? QB : 1][16];  // dbias values a later member adds to (see below)
    auto qblock = [&](const char* sb, int q0t, int qb, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // dp starts at -D of the 16 queries this lane holds (rows res_row(g, h) of the block:
      // register g of the 32x32 result is row 8(g/4) + 4h + g%4, four consecutive rows per
      // 16-byte read), so the dP MFMA chain delivers dP - D
      f32x16 sc = f32x16{}, dp;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 nd = *reinterpret_cast<const f32x4*>(sb + L::DLT + (32 * qb + 8 * q4 + 4 * h) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * q4 + e] = nd[e];
      }
      {
        u32x4 qa[DK], da[DK];
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          qa[ks] = lds_ld16(sb + L::QT, 32 * qb * RB + ra[ks]);
          da[ks] = lds_ld16(sb + L::DT, 32 * qb * RB + ra[ks]);
        }
        sched_fence();  // all Q and dO operands in flight before the first MFMA
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
          sc = E::mma(qa[ks], kf[ks], sc);
          dp = E::mma(da[ks], vf[ks], dp);
        }
      }
      // LSE * log2(e) of the 16 queries this lane holds
      f32x4 l4[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = 32 * qb + 8 * q4 + 4 * h;
        l4[q4] = *reinterpret_cast<const f32x4*>(sb + L::LSE + r0 * 4);
      }
      float p[16], ds[16], adist[BIAS ? 16 : 1];
      const char* bs = sb + L::STAGE + wid_s * BT::kWaveBytes;  // this wave's bias windows
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const float lq = l4[g / 4][g % 4];  // already in log2 units
        float x;
        if constexpr (TENSOR) {
          x = __builtin_fmaf(sc[g], sl2, __builtin_fmaf(BT::read(bs, qb, g, lane), kLog2e, -lq));
        } else if constexpr (BIAS) {
          const float dist = (float)(q0t + 32 * qb + 4 * h - key) + (float)(8 * (g / 4) + (g % 4));
          adist[g] = __builtin_fabsf(dist);
          x = __builtin_fmaf(sc[g], sl2, __builtin_fmaf(slope2, adist[g], -lq));
        } else {
          x = __builtin_fmaf(sc[g], sl2, -lq);
        }
        p[g] = fast_exp2(x);
      }
      if constexpr (MASK) {
        int4 st4[4], en4[4];
        if (ranged) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int r0 = 32 * qb + 8 * q4 + 4 * h;
            st4[q4] = *reinterpret_cast<const int4*>(sb + L::KS + r0 * 4);
            en4[q4] = *reinterpret_cast<const int4*>(sb + L::KE + r0 * 4);
          }
        }
        const int kvis = key < Nk ? 1 : 0;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int qi = q0t + 32 * qb + res_row(g, h);
          const int lo = ranged ? min(max((&st4[g / 4].x)[g % 4], 0), Nk) : 0;
          const int hi = ranged ? min(max((&en4[g / 4].x)[g % 4], 0), Nk) : Nk;
          const int cmin = causal ? qi + off : Nk;
          const bool vis = kvis && qi < Nq && key >= lo && key < hi && key <= cmin;
          p[g] = vis ? p[g] : 0.f;
        }
      }
#pragma unroll
      for (int g = 0; g < 16; ++g) ds[g] = p[g] * dp[g];  // dp holds dP - D
      if constexpr (DQA) {
        // dS^T row 32 w + n (this lane's key), queries 32 qb + 8 t4 + 4 h + (0..3)
        const int rr = 32 * wid_s + n;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
          lds_st8(dsw, rr * (2 * BR) + 16 * ((4 * qb + t4) ^ swz<64>(rr)) + 8 * h,
                  u32x2{E::pack2(ds[4 * t4], ds[4 * t4 + 1]),
                        E::pack2(ds[4 * t4 + 2], ds[4 * t4 + 3])});
      }
      if constexpr (TENSOR) {
        // dbias = dS (zero where masked: p = 0 there); lanes 0-31 and 32-63 each store 128
        // contiguous bytes of one row. Rows summed: the lane adds its 16 rows.
        if (dB != nullptr && key < Nk) {
          if (rrows) {
#pragma unroll
            for (int g = 0; g < 16; ++g) dbr += ds[g];
          } else {
#pragma unroll
            for (int g = 0; g < 16; ++g) {
              const int qi = q0t + 32 * qb + res_row(g, h);
              if (qi < Nq) {
                float* pd = dB + (size_t)qi * Nk + key;
                *pd = first ? ds[g] : pre[qb][g] + ds[g];
              }
            }
          }
        }
      }
      if constexpr (BIAS) {
        // the slope's gradient: dS |i - j| over the visible entries (masked ones have p = 0)
#pragma unroll
        for (int g = 0; g < 16; ++g) sgrad = __builtin_fmaf(ds[g], adist[g], sgrad);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 pa, dsa;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pa[w] = E::pack2(p[8 * st + 2 * w], p[8 * st + 2 * w + 1]);
          dsa[w] = E::pack2(ds[8 * st + 2 * w], ds[8 * st + 2 * w + 1]);
        }
        u32x4 ob[DB], qbf[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          ob[db] = cfrag(sb + L::DT, qb, st, db);
          qbf[db] = cfrag(sb + L::QT, qb, st, db);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = E::mma(pa, ob[db], dv[db]);
          dk[db] = E::mma(dsa, qbf[db], dk[db]);
        }
      }
    };

    // ---- ring of ST stages, P = ST-1 query tiles in flight -------------------------------
    Tile tile_ld;
    tile_ld.init(wid_s, lane);
    // wave w brings the tile's row array w: 0 LSE*log2(e), 1 D, 2 key_start, 3 key_end
    // (without a range mask waves 2 and 3 load the first array again, so that every wave
    // issues the same count)
    const float* arr_base;
    {
      const float* lse_h = a.lse2 + (size_t)bh * Nq;  // LSE * log2(e), from the prep pass
      const float* dlt_h = a.delta + (size_t)bh * Nq;
      arr_base = wid_s == 0 ? lse_h : wid_s == 1 ? dlt_h
               : ranged ? reinterpret_cast<const float*>(wid_s == 2 ? a.key_start : a.key_end) : lse_h;
    }
    const int arr_off = wid_s == 0 ? L::LSE : wid_s == 1 ? L::DLT : wid_s == 2 ? L::KS : L::KE;
    // ring position p (query tile tile_at(p)) lives in stage p % ST
    auto stage_of = [&](int p) { return smem + (p % ST) * kStage; };
    auto issue = [&](int p) {
      char* sb = stage_of(p);
      const int q0t = tile_at(p) * BR;
      tile_ld.template load<false>(Q, q0t, Nq, sb + L::QT, wid_s);
      tile_ld.template load<false>(dO, q0t, Nq, sb + L::DT, wid_s);
      dma4<false>(arr_base, (uint32_t)min(q0t + lane, Nq - 1), sb + arr_off);
      if constexpr (TENSOR)
        BT::load(TB, a.tb_si, q0t, Nq, kw0, Nk, sb + L::STAGE + wid_s * BT::kWaveBytes, lane);
    };
    auto land = [&](int later) {
      if (P >= 3 && later >= 3) wait_vmem<(P >= 3 ? 3 : 0) * kOpsPerTile>();
      else if (P >= 2 && later == 2) wait_vmem<(P >= 2 ? 2 : 0) * kOpsPerTile>();
      else if (later == 1) wait_vmem<kOpsPerTile>();
      else wait_vmem<0>();
      if constexpr (DQA) __syncthreads();  // the dS^T stores too
      else __builtin_amdgcn_s_barrier();
    };
    // dQ of ring position pp from its dS^T (written by every wave before the barrier that
    // ended that position): 8 products over 16 keys each per 32-row block, then one
    // float32 atomic add per element into dq
    auto dq_tile = [&](int pp) {
      const char* dsr = dst_s + (pp & 1) * kDsBuf;
      const int q0p = tile_at(pp) * BR;
      float* dqp = static_cast<float*>(a.dq) + (size_t)bh * Nq * D + 32 * dbw + n;
      for (int u = wid_s; u < DB * QB; u += NW) {
        const int qb = u / DB;
        int oa[2];
#pragma unroll
        for (int pp2 = 0; pp2 < 2; ++pp2) {
          const int r = 8 * pp2 + 4 * h + q4;
          oa[pp2] = r * (2 * BR) + 16 * ((4 * qb + 2 * g16 + (lo2 >> 1)) ^ swz<64>(r)) +
                    8 * (lo2 & 1);
        }
        u32x4 af[NS];
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) {
          const u32x2 lo = lds_ld8_tr(dsr, 16 * s2 * (2 * BR) + oa[0]);
          const u32x2 hi = lds_ld8_tr(dsr, 16 * s2 * (2 * BR) + oa[1]);
          af[s2] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
        sched_fence();
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) acc = E::mma(af[s2], kt[s2], acc);
        const float scale = a.scale;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int qi = q0p + 32 * qb + res_row(g, h);
          if (qi < Nq) unsafeAtomicAdd(dqp + (size_t)qi * D, acc[g] * scale);
        }
      }
    };
    // zero dbias of query tile t for this wave's keys (lanes 0-31 and 32-63: alternate rows)
    // (only the first member: later ones add nothing there; rows summed: written at the end)
    // (with a bitmap the launch clears dbias first: tiles no wave lists are never visited)
    auto zero_dbias_tile = [&](int t) {
      if (SPARSE || dB == nullptr || rrows || !first || key >= Nk) return;
      for (int i = 0; i < BR / 2; ++i) {
        const int qi = t * BR + 2 * i + h;
        if (qi < Nq) dB[(size_t)qi * Nk + key] = 0.f;
      }
    };
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (i < n_pos) issue(i);
    // The K and V fragments and every prologue tile land here. Waiting for all of them
    // (rather than for the first tile only) leaves no register load outstanding once the
    // loop starts, so the compiler has no reason to put a full vector-memory wait, which
    // would also wait for the ring's loads in flight, in front of the loop's MFMAs.
    wait_vmem<0>();
    __builtin_amdgcn_s_barrier();

    for (int p = 0; p < n_pos; ++p) {
#pragma unroll
      for (int db = 0; db < DB; ++db) { pin_agpr(dv[db]); pin_agpr(dk[db]); }
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) { pin_agpr(kf[ks]); pin_agpr(vf[ks]); }
      // the stage of position p+P held position p-1, which every wave finished before the
      // barrier
      if constexpr (SPARSE) lw.slide(p);
      if (p + P < n_pos) issue(p + P);
      sync_check();
      if constexpr (DQA) {
        if (p > 0) dq_tile(p - 1);
        dsw = dst_s + (p & 1) * kDsBuf;
      }
      const int t = tile_at(p);
      const int q0t = t * BR;
      const char* sb = stage_of(p);

      // classify the tile for this wave's keys [kw0, kw1)
      bool skip = kw0 >= Nk;
      bool full = q0t + BR <= Nq && kw0 + 32 <= Nk;
      if (causal) {
        skip |= q0t + BR - 1 + off < kw0;
        full &= q0t + off >= kw0 + 31;
      }
      if (ranged) {
        // tile t's summary through the constant address space: a scalar load, whose wait
        // does not cover the ring's loads in flight (a vector load here made every tile wait
        // for the tile just issued)
        const __attribute__((address_space(4))) int* sm =
            (const __attribute__((address_space(4))) int*)a.qsum + 4 * t;
        skip |= kw1 <= sm[0] || kw0 >= sm[3];
        full &= sm[1] <= kw0 && sm[2] >= kw0 + 32;
      }
      if constexpr (SPARSE) skip = !((lw.at(p) >> (16 + wid_s)) & 1u);
      if constexpr (TENSOR) {
        // later members add to dbias: read the values this lane adds to before the tile's
        // products, so the loads' latency hides behind them
        if (!skip && !first && !rrows && dB != nullptr && key < Nk) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int g = 0; g < 16; ++g) {
              const int qi = min(q0t + 32 * qb + res_row(g, h), Nq - 1);
              pre[qb][g] = dB[(size_t)qi * Nk + key];
            }
        }
      }
      if (!skip) {
        if (full) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) qblock(sb, q0t, qb, std::false_type{});
        } else {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) qblock(sb, q0t, qb, std::true_type{});
        }
      } else if constexpr (TENSOR) {
        zero_dbias_tile(t);
      }
      if constexpr (DQA) {
        if (skip) {  // no key of this wave visible: its dS^T rows are zero
          const int rr = 32 * wid_s + (lane >> 1);
#pragma unroll
          for (int j = 0; j < 4; ++j) lds_st16(dsw, rr * (2 * BR) + 64 * (lane & 1) + 16 * j, u32x4{});
        }
      }
      if (p + 1 < n_pos) land(min(p + P, n_pos - 1) - (p + 1));
    }
    if constexpr (DQA) {
      if (n_pos > 0) {
        __syncthreads();
        dq_tile(n_pos - 1);
      }
    }
    // dbias of the query tiles outside the workgroup's window is zero (every (i, j) of this
    // wave's keys is then written exactly once: computed, or zero where nothing is visible)
    if constexpr (TENSOR) {
      if (dB != nullptr) {
        for (int t = 0; t < t_lo; ++t) zero_dbias_tile(t);
        for (int t = max(t_hi, t_lo); t < nqt; ++t) zero_dbias_tile(t);
      }
    }

    // the workgroup's partial of dL/dslope (every workgroup writes one, zero if it saw
    // nothing, so the reduction reads only values of this call)
    if constexpr (BIAS) {
      if (a.dslope_part != nullptr) {
        __shared__ float sred[NW];
        const float w = wave_fsum(sgrad);
        if (lane == 0) sred[wid_s] = w;
        __syncthreads();
        if (tid == 0) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < NW; ++i) acc += sred[i];
          a.dslope_part[(size_t)bh * a.nblk + kb] = acc;
        }
      }
    }

    // epilogue: lane holds column d = 32*db + n for keys kw0 + res_row(g, h)
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int kr = kw0 + res_row(g, h);
        if (kr < Nk) {
          const size_t idx = ((size_t)bh * Nk + kr) * D + 32 * db + n;
          if (a.grad_f32) {
            static_cast<float*>(a.dk)[idx] = dk[db][g] * scale;
            static_cast<float*>(a.dv)[idx] = dv[db][g];
          } else {
            static_cast<T*>(a.dk)[idx] = (T)(dk[db][g] * scale);
            static_cast<T*>(a.dv)[idx] = (T)dv[db][g];
          }
        }
      }
    }
    // rows summed: the two lanes of a key hold the sums of alternate row groups
    if constexpr (TENSOR) {
      if (rrows && dB != nullptr && m == n_mem - 1) {
        const float tot = dbr + __shfl_xor(dbr, 32, 64);
        if (h == 0 && key < Nk) dB[key] = tot;
      }
    }
  }  // members
}

// ---------------------------------------------------------------------------------
// 3. dQ: query-block-outer
// ---------------------------------------------------------------------------------
// Per stage: K and V tiles (BC rows each, swizzled, filled by direct loads). K is read
// both ways: 16-byte rows (A operand of S^T = K Q^T) and transposing gathers (A operand
// of dQ^T += K^T dS^T); V rows are the A operand of dP^T = V dO^T.
template <int D, int BC>
struct DqLds {
  static constexpr int RB = 2 * D;
  static constexpr int KT = 0, VT = BC * RB;
  static constexpr int STAGE = 2 * BC * RB;
};

#ifndef FA_DQ_STAGES
#define FA_DQ_STAGES 4
#endif

template <typename T, int D, int BC, int NW, int WPE, int BM, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dq_kernel(const BwdArgs a) {
  using E = Elt<T>;
  using L = DqLds<D, BC>;
  using Tile = DmaTile<BC, D, NW>;
  constexpr bool BIAS = BM == kBiasSlope, TENSOR = BM == kBiasTensor;
  using BT = BiasRowTile<TENSOR ? BC : 64>;
  constexpr int BRQ = 32 * NW, KB = BC / 32, DK = D / 16, DB = D / 32, RB = L::RB;
  // the bias tensor's tile (32 rows x BC float32 per wave) leaves room for two stages
  constexpr int ST = TENSOR ? 2 : FA_DQ_STAGES, P = ST - 1;
  constexpr int kOpsPerTile = 2 * Tile::kOpsPerWave + (TENSOR ? BT::kOps : 0);
  constexpr int kStage = L::STAGE + (TENSOR ? NW * BT::kWaveBytes : 0);
  static_assert(P * kOpsPerTile < 64, "vmcnt range");
  static_assert(ST * kStage <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[ST * kStage];
  __shared__ int wg_win[NW][2];

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id(), n = lane & 31, h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const bool causal = a.causal != 0, ranged = a.key_start != nullptr;
  int bh, qb;
  map_block(blockIdx.x, a.B * a.H, a.nblk, a.sched, true, bh, qb);
  const int head = bh % a.H;
  const T* Q = static_cast<const T*>(a.q) + (size_t)bh * Nq * D;
  const T* K = static_cast<const T*>(a.k) + (size_t)bh * Nk * D;
  const T* V = static_cast<const T*>(a.v) + (size_t)bh * Nk * D;
  const T* dO = static_cast<const T*>(a.dout) + (size_t)bh * Nq * D;
  const float sl2 = a.sl2;
  const float slope2 = BIAS ? a.slope2[a.n_slopes == 1 ? 0 : head] : 0.f;
  const float* TB = TENSOR ? a.tbias + (long long)(bh / a.H) * a.tb_sb + (long long)head * a.tb_sh
                           : nullptr;

  const int q0 = qb * BRQ, wq0 = q0 + 32 * wid;
  const int qrow = wq0 + n;
  const size_t qr = (size_t)min(qrow, Nq - 1);
  u32x4 qf[DK], dof[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    qf[ks] = ldg16(Q + qr * D + 16 * ks + 8 * h);
    dof[ks] = ldg16(dO + qr * D + 16 * ks + 8 * h);
  }
  const float lq = lse_offset2(a.lse[(size_t)bh * Nq + qr]);
  // -D of this lane's query row (the prep pass stores D negated). Starting the dP^T
  // accumulation from it, as the dK/dV pass does, would keep 16 more registers live and
  // spill at this kernel's 256.
  const float nd = a.delta[(size_t)bh * Nq + qr];

  // key window of this wave / workgroup (same rules as the forward pass)
  int kst = 0, ken = Nk;
  // wave-uniform summaries of the rows' key intervals (rows past the end take no part);
  // computed inside the uniform branch so they stay scalar
  int w_min_s = Nk, w_max_s = 0, w_min_e = Nk, w_max_e = 0;
  if (ranged) {
    const bool in = qrow < Nq;
    if (in) {
      kst = min(max(a.key_start[qrow], 0), Nk);
      ken = min(max(a.key_end[qrow], 0), Nk);
    }
    w_min_s = wave_min(in ? kst : Nk);
    w_max_s = wave_max(in ? kst : 0);
    w_min_e = wave_min(in ? ken : Nk);
    w_max_e = wave_max(in ? ken : 0);
  }
  const bool wave_live = wq0 < Nq;
  const int wq_last = min(wq0 + 32, Nq) - 1;
  int w_lo = 0, w_hi = Nk, w_full_c = Nk;
  if (causal) {
    w_hi = min(w_hi, wq_last + off + 1);
    w_full_c = max(0, min(Nk, wq0 + off + 1));
  }
  if (ranged) {
    w_lo = max(w_lo, w_min_s);
    w_hi = min(w_hi, w_max_e);
  }
  if (!wave_live || w_hi <= w_lo) { w_lo = Nk; w_hi = 0; }
  if (lane == 0) { wg_win[wid][0] = w_lo; wg_win[wid][1] = w_hi; }
  __syncthreads();
  int g_lo = Nk, g_hi = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { g_lo = min(g_lo, wg_win[w][0]); g_hi = max(g_hi, wg_win[w][1]); }
  const int t_lo = g_hi > g_lo ? g_lo / BC : 0;
  const int t_hi = g_hi > g_lo ? (g_hi + BC - 1) / BC : 0;

  // block-sparse bitmap: the key tiles the workgroup loads (see build_tile_list); with
  // 64-key tiles a tile and a wave's 32 rows each lie inside one block
  constexpr int kMaxT = SPARSE ? FA_MAX_SPARSE_N / BC : 64;
  static_assert(!SPARSE || BC == 64, "block-sparse dQ uses 64-key tiles");
  __shared__ uint32_t need_w[SPARSE ? NW : 1][2 * (kMaxT / 64)];
  __shared__ uint32_t tlist[SPARSE ? kMaxT : 1];
  __shared__ int n_list_s;
  int n_pos = t_hi - t_lo;
  if constexpr (SPARSE) {
    const uint8_t* brow = nullptr;
    if (wave_live) {
      const int bb = bh / a.H, hh = bh - bb * a.H;
      brow = a.bmask + bb * a.bm_sb + hh * a.bm_sh + (long long)(wq0 / a.bq) * a.nkb;
    }
    n_pos = build_tile_list(need_w, tlist, &n_list_s, wid, lane, t_lo, t_hi, [&](int t) {
      const int kt0 = t * BC;
      return brow != nullptr && !(kt0 >= w_hi || kt0 + BC <= w_lo) && brow[kt0 / a.bk] != 0;
    });
  }
  ListWindow<kMaxT> lw;
  if constexpr (SPARSE) lw.init(tlist, lane);
  auto tile_at = [&](int p) -> int {
    if constexpr (SPARSE) return (int)(lw.at(p) & 0xffffu);
    else return t_lo + p;
  };

  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};

  // LDS offsets inside a swizzled tile: row reads of key row 32kb + n, chunk 2ks + h;
  // transposing gathers of 8 keys of one d column (K^T fragments).
  int ra[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) ra[ks] = n * RB + 16 * ((2 * ks + h) ^ swz<D>(n));
  int ta[DB][2];
  {
    const int q = (lane >> 2) & 3, g16 = (lane >> 4) & 1, lo2 = lane & 3;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 8 * p + 4 * h + q;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        ta[db][p] = r * RB + 16 * ((4 * db + 2 * g16 + (lo2 >> 1)) ^ swz<D>(r)) + 8 * (lo2 & 1);
    }
  }
  auto ktfrag = [&](const char* Ks, int kb, int st, int db) {
    const int rows = (32 * kb + 16 * st) * RB;
    const u32x2 lo = lds_ld8_tr(Ks, rows + ta[db][0]);
    const u32x2 hi = lds_ld8_tr(Ks, rows + ta[db][1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  auto tile = [&](const char* sb, int kt0, bool masked) __attribute__((always_inline)) {
    const char* Ks = sb + L::KT;
    const char* Vs = sb + L::VT;
    f32x16 sc[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // each batch of 8 operands is in flight before its MFMAs (fenced), one batch of
      // registers at a time
      {
        u32x4 ka[DK];
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) ka[ks] = lds_ld16(Ks, kb * 32 * RB + ra[ks]);
        sched_fence();
        sc[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) sc[kb] = E::mma(ka[ks], qf[ks], sc[kb]);
      }
      {
        u32x4 va[DK];
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) va[ks] = lds_ld16(Vs, kb * 32 * RB + ra[ks]);
        sched_fence();
        dp[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) dp[kb] = E::mma(va[ks], dof[ks], dp[kb]);
      }
    }
    const char* Bs = sb + L::STAGE + wid * BT::kWaveBytes;  // this wave's bias rows
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x4 bv[TENSOR ? 4 : 1];
      if constexpr (TENSOR) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) bv[g4] = BT::read(Bs, n, kb * 32 + 8 * g4 + 4 * h);
      }
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        float x;
        if constexpr (TENSOR) {
          x = __builtin_fmaf(sc[kb][g], sl2, __builtin_fmaf(bv[g / 4][g % 4], kLog2e, -lq));
        } else if constexpr (BIAS) {
          const float dist = (float)(qrow - kt0 - 4 * h) - (float)(kb * 32 + 8 * (g / 4) + (g % 4));
          x = __builtin_fmaf(sc[kb][g], sl2, __builtin_fmaf(slope2, __builtin_fabsf(dist), -lq));
        } else {
          x = __builtin_fmaf(sc[kb][g], sl2, -lq);
        }
        sc[kb][g] = fast_exp2(x);
      }
      if (masked) {
        // tile-local visible keys [lo, hi) of this row; register g holds key
        // kb*32 + res_row(g, h) = c + 4h (c constant), so the bounds are shifted by 4h
        const int hi4 = min(min(ken, Nk), causal ? qrow + off + 1 : Nk) - kt0 - 4 * h;
        if (ranged) {
          const int lo4 = kst - kt0 - 4 * h;
          const unsigned span = (unsigned)max(hi4 - lo4, 0);  // c visible iff c - lo4 < span
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const int c = kb * 32 + res_row(g, 0);
            sc[kb][g] = (unsigned)(c - lo4) < span ? sc[kb][g] : 0.f;
          }
        } else {
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const int c = kb * 32 + res_row(g, 0);
            sc[kb][g] = c < hi4 ? sc[kb][g] : 0.f;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < 16; ++g) sc[kb][g] = sc[kb][g] * (dp[kb][g] + nd);  // dS^T
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 da;
#pragma unroll
        for (int w = 0; w < 4; ++w) da[w] = E::pack2(sc[kb][8 * st + 2 * w], sc[kb][8 * st + 2 * w + 1]);
        u32x4 kt[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) kt[db] = ktfrag(Ks, kb, st, db);
#pragma unroll
        for (int db = 0; db < DB; ++db) dqa[db] = E::mma(kt[db], da, dqa[db]);
      }
    }
  };

  Tile tile_ld;
  tile_ld.init(wid, lane);
  // ring position p (key tile tile_at(p)) lives in stage p % ST
  auto stage_of = [&](int p) { return smem + (p % ST) * kStage; };
  auto issue = [&](int p) {
    char* sb = stage_of(p);
    const int t = tile_at(p);
    tile_ld.load(K, t * BC, Nk, sb + L::KT, wid);
    tile_ld.load(V, t * BC, Nk, sb + L::VT, wid);
    if constexpr (TENSOR)
      BT::load(TB, a.tb_si, wq0, Nq, t * BC, Nk, sb + L::STAGE + wid * BT::kWaveBytes, lane);
  };
  auto land = [&](int later) {
    if (P >= 3 && later >= 3) wait_vmem<(P >= 3 ? 3 : 0) * kOpsPerTile>();
    else if (P >= 2 && later == 2) wait_vmem<(P >= 2 ? 2 : 0) * kOpsPerTile>();
    else if (later == 1) wait_vmem<kOpsPerTile>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
  };
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (i < n_pos) issue(i);
  if (0 < n_pos) land(min(P, n_pos) - 1);
  for (int p = 0; p < n_pos; ++p) {
    // the stage of position p+P held position p-1, which every wave finished before the
    // barrier
    if constexpr (SPARSE) lw.slide(p);
    if (p + P < n_pos) issue(p + P);
    sync_check();
    const int t = tile_at(p);
    const int kt0 = t * BC, kt1 = kt0 + BC;
    bool skip = kt0 >= w_hi || kt1 <= w_lo;
    if constexpr (SPARSE) skip = !((lw.at(p) >> (16 + wid)) & 1u);
    if (!skip) {
      const bool full = kt1 <= Nk && kt1 <= w_full_c &&
                        (!ranged || (w_max_s <= kt0 && w_min_e >= kt1));
      tile(stage_of(p), kt0, !full);
    }
    if (p + 1 < n_pos) land(min(p + P, n_pos - 1) - (p + 1));
  }

  // epilogue: lane holds query qrow, registers d = 32*db + res_row(g, h)
  if (qrow < Nq) {
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * h;
        store_grad4<T>(a.dq, ((size_t)bh * Nq + qrow) * D + d0, a.grad_f32 != 0,
                       dqa[db][4 * g4] * scale, dqa[db][4 * g4 + 1] * scale,
                       dqa[db][4 * g4 + 2] * scale, dqa[db][4 * g4 + 3] * scale);
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------------

size_t bwd_qsum_offset(int B, int H, int Nq) {
  return (((size_t)B * H * Nq * sizeof(float)) + 255) & ~(size_t)255;
}
size_t bwd_lse2_offset(int B, int H, int Nq) {
  const size_t nt = (size_t)(Nq + kDkdvBR - 1) / kDkdvBR;
  return bwd_qsum_offset(B, H, Nq) + ((nt * 4 * sizeof(int32_t) + 255) & ~(size_t)255);
}
size_t bwd_dslope_offset(int B, int H, int Nq) {
  return bwd_lse2_offset(B, H, Nq) + (((size_t)B * H * Nq * sizeof(float) + 255) & ~(size_t)255);
}
size_t bwd_workspace_bytes(int B, int H, int Nq, int Nk) {
  const size_t nblk = (size_t)(Nk + 32 * 4 - 1) / (32 * 4);  // key blocks of the dK/dV pass
  return bwd_dslope_offset(B, H, Nq) + (((size_t)B * H * nblk * sizeof(float) + 255) & ~(size_t)255);
}

// dL/dslope from the dK/dV pass's per-workgroup partials, one thread per slope, summed in
// a fixed order (batch, then key block; all heads for a shared slope)
static __global__ void dslope_reduce_kernel(const float* __restrict__ part, int B, int H, int nblk,
                                     int n_slopes, float* __restrict__ out) {
  const int s = threadIdx.x;
  if (s >= n_slopes) return;
  const int h0 = n_slopes == 1 ? 0 : s, h1 = n_slopes == 1 ? H : s + 1;
  float acc = 0.f;
  for (int b = 0; b < B; ++b)
    for (int h = h0; h < h1; ++h)
      for (int k = 0; k < nblk; ++k) acc += part[((size_t)b * H + h) * nblk + k];
  out[s] = acc;
}

// Clears n floats (a dense dbias before a block-sparse dK/dV pass writes the visible
// entries; a kernel rather than a memset node, so that a captured graph replays it
// correctly).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0.f;
}

// Clears n4 float4 (dq before the dK/dV pass adds into it with atomics; a kernel rather
// than a memset node, so that a captured graph replays it correctly).
__global__ __launch_bounds__(256) void zero_f32x4_kernel(f32x4* __restrict__ p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256)
    p[i] = f32x4{};
}

template <typename T, int D, int DKDV_NW, int DKDV_WPE, int DQ_BC, int DQ_NW, int DQ_WPE>
static hipError_t launch_bwd_t(int bias, int phases, BwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int rows = BH * a.Nq;
  constexpr int RPB = 256 / (D / 8);
  hipError_t e = hipSuccess;
  if (phases & FA_BWD_PREP) {
    hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                       static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.lse, a.delta,
                       a.lse2, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.key_start != nullptr) {
      e = launch_mask_summary(a.key_start, a.key_end, a.Nq, a.Nk, kDkdvBR, a.qsum, st);
      if (e != hipSuccess) return e;
    }
  }
  const int sched = (BH % 8 == 0) ? kSchedXcdLpt : kSchedHeadMajor;
  // dK, dV
  if (phases & FA_BWD_DKDV) {
    constexpr int BK = 32 * DKDV_NW;
    BwdArgs b = a;
    b.nblk = (a.Nk + BK - 1) / BK;
    // a workgroup per dbias slice and key block: dbias summed over batches or heads
    // makes one workgroup compute every (b, h) of its slice
    int slots = BH;
    if (bias == kBiasTensor && a.dbias != nullptr)
      slots = ((a.db_red & FA_DBIAS_SUM_BATCH) ? 1 : a.B) *
              ((a.db_red & FA_DBIAS_SUM_HEADS) ? 1 : a.H);
    else
      b.db_red = 0;
    b.sched = (slots % 8 == 0) ? 1 : 0;
    const dim3 grid((unsigned)(slots * b.nblk)), block(DKDV_NW * 64);
    const bool sparse = a.bmask != nullptr;
    if (phases & FA_BWD_DQ_ATOMIC) {
      const size_t n4 = (size_t)BH * a.Nq * D / 4;
      const unsigned zb = (unsigned)std::min<size_t>((n4 + 255) / 256, 4096);
      hipLaunchKernelGGL(zero_f32x4_kernel, dim3(zb), dim3(256), 0, st,
                         static_cast<f32x4*>(a.dq), n4);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (phases & FA_BWD_DQ_ATOMIC) {
      if (bias)
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasSlope, false, false, true>), grid, block, 0, st, b);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasNone, false, false, true>), grid, block, 0, st, b);
    } else if (bias == kBiasTensor && slots != BH && sparse) {
      // dbias summed over batches or heads with a bitmap: cleared first, every member adds
      if ((a.db_red & FA_DBIAS_SUM_ROWS) == 0) {
        const size_t nd = (size_t)slots * a.Nq * a.Nk;
        const unsigned zb = (unsigned)std::min<size_t>((nd + 255) / 256, 8192);
        hipLaunchKernelGGL(zero_f32_kernel, dim3(zb), dim3(256), 0, st, a.dbias, nd);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasTensor, true, true>), grid, block, 0, st, b);
    } else if (bias == kBiasTensor && slots != BH) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasTensor, false, true>), grid, block, 0, st, b);
    } else if (bias == kBiasTensor && sparse) {
      // a dense dbias is cleared first: tiles no wave of a workgroup lists are never
      // visited, so the kernel does not write their zeros itself
      if (a.dbias != nullptr && (a.db_red & FA_DBIAS_SUM_ROWS) == 0) {
        const size_t nd = (size_t)BH * a.Nq * a.Nk;
        const unsigned zb = (unsigned)std::min<size_t>((nd + 255) / 256, 8192);
        hipLaunchKernelGGL(zero_f32_kernel, dim3(zb), dim3(256), 0, st, a.dbias, nd);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasTensor, true>), grid, block, 0, st, b);
    } else if (bias == kBiasTensor) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasTensor, false>), grid, block, 0, st, b);
    }
    else if (bias && sparse)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasSlope, true>), grid, block, 0, st, b);
    else if (bias)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasSlope, false>), grid, block, 0, st, b);
    else if (sparse)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasNone, true>), grid, block, 0, st, b);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, kDkdvBR, DKDV_NW, DKDV_WPE, kBiasNone, false>), grid, block, 0, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bias == kBiasSlope && a.dslopes != nullptr) {
      e = launch_dslope_reduce(b.dslope_part, a.B, a.H, b.nblk, a.n_slopes, a.dslopes, st);
      if (e != hipSuccess) return e;
    }
  }
  // dQ
  if (phases & FA_BWD_DQ) {
    // the bias tensor's form: 4 waves, 64-key tiles, two stages (its tile shares them)
    const int nw = bias == kBiasTensor ? 4 : DQ_NW;
    const int brq = 32 * nw;
    BwdArgs b = a;
    b.nblk = (a.Nq + brq - 1) / brq;
    b.sched = sched;
    const dim3 grid((unsigned)(BH * b.nblk)), block(nw * 64);
    // (the block-sparse form always uses 64-key tiles, which lie inside one block)
    if (bias == kBiasTensor && a.bmask != nullptr)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, 64, 4, DQ_WPE, kBiasTensor, true>), grid, block, 0, st, b);
    else if (bias == kBiasTensor)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, 64, 4, DQ_WPE, kBiasTensor, false>), grid, block, 0, st, b);
    else if (a.bmask != nullptr && bias)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, 64, DQ_NW, DQ_WPE, kBiasSlope, true>), grid, block, 0, st, b);
    else if (a.bmask != nullptr)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, 64, DQ_NW, DQ_WPE, kBiasNone, true>), grid, block, 0, st, b);
    else if (bias)
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, DQ_BC, DQ_NW, DQ_WPE, kBiasSlope, false>), grid, block, 0, st, b);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, DQ_BC, DQ_NW, DQ_WPE, kBiasNone, false>), grid, block, 0, st, b);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd(fa_dtype dt, int d, int bias, int phases, BwdArgs& a, hipStream_t st) {
  switch (dt) {
    case FA_BF16:
      return d == 128 ? launch_bwd_t<__bf16, 128, 4, 1, 64, 8, 2>(bias, phases, a, st)
                      : launch_bwd_t<__bf16, 64, 4, 1, 128, 8, 2>(bias, phases, a, st);
    case FA_F16:
      return d == 128 ? launch_bwd_t<_Float16, 128, 4, 1, 64, 8, 2>(bias, phases, a, st)
                      : launch_bwd_t<_Float16, 64, 4, 1, 128, 8, 2>(bias, phases, a, st);
    case FA_F32:
      return launch_bwd32(d, bias, phases, a, st);
    default:
      return hipErrorNotSupported;
  }
}

hipError_t launch_dslope_reduce(const float* part, int B, int H, int nblk, int n_slopes,
                                float* out, hipStream_t st) {
  hipLaunchKernelGGL(dslope_reduce_kernel, dim3(1), dim3(FA_MAX_SLOPES), 0, st, part, B, H, nblk,
                     n_slopes, out);
  return hipGetLastError();
}

}  // namespace fa
