// Backward pass for float32 inputs: the same recomputation as the 16-bit kernels (D =
// rowsum(dO * O); a key-outer pass recomputing S and P per query tile for dV = P^T dO and
// dK = scale dS^T Q; a query-outer pass recomputing them per key tile for dQ = scale dS K),
// with every product on v_mfma_f32_32x32x2_f32 and no rounding of P or dS.
//
// Source: marketmaker.cc attention page, the section on the backward pass recomputing
// rather than storing (only O and the per-row statistics are kept from the forward);
// masks and bias as in the forward (its causal-masking section; the scifaro.com
// related-papers page for FlashMask on an additive bias matrix).
//
// Operand layouts of the 32x32x2 float32 MFMA: A[i][k] comes from lane i + 32 k, B[k][j]
// from lane j + 32 k, and lane j + 32 h ends with C[res_row(g, h)][j] for g < 16. A
// product over a 32-row block of the contraction index therefore takes 16 steps g, step g
// pairing rows res_row(g, 0) and res_row(g, 1): exactly the two values lanes j and j + 32
// hold in register g of a previous result, so P (and dS) feed the next products from
// registers. Each pass holds one operand side in registers (K and V of the wave's keys,
// or Q and dO of the wave's queries) and reads the other from LDS tiles whose rows are
// padded to d + 2 floats (the 16-byte-apart reads of 32 consecutive rows then cover all
// 64 banks).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

// D = rowsum(dO * O) and the row's exponent offset (LSE * log2(e); +inf for an empty row)
template <int D>
__global__ __launch_bounds__(256) void prep32_kernel(const float* __restrict__ o,
                                                     const float* __restrict__ dout,
                                                     const float* __restrict__ lse,
                                                     float* __restrict__ delta,
                                                     float* __restrict__ lse2, int rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 floats each
  constexpr int RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + (int)threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const f32x4* po = reinterpret_cast<const f32x4*>(o + (size_t)row * D + 8 * c);
    const f32x4* pd = reinterpret_cast<const f32x4*>(dout + (size_t)row * D + 8 * c);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 x = po[j], y = pd[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(x[e], y[e], acc);
    }
  }
#pragma unroll
  for (int s = TPR / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (row < rows && c == 0) {
    delta[row] = acc;
    lse2[row] = lse_offset2(lse[row]);
  }
}

__device__ inline f32x16 mma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// One 32-row tile of two row-major float32 matrices (rows past the end repeat the last
// row) through registers into LDS rows of RS floats: 256 threads, float4 loads, 8-byte
// LDS stores (RS is even).
template <int D, int RS>
struct Tile32 {
  static constexpr int kPer = 32 * D / 4 / 256;  // float4 per thread and matrix
  f32x4 r0[kPer], r1[kPer];
  __device__ inline void load(const float* m0, const float* m1, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 4), col = c % (D / 4);
      const size_t r = (size_t)min(row0 + row, nrows - 1);
      r0[i] = *reinterpret_cast<const f32x4*>(m0 + r * D + 4 * col);
      r1[i] = *reinterpret_cast<const f32x4*>(m1 + r * D + 4 * col);
    }
  }
  __device__ inline void store(float* s0, float* s1, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / 4), col = c % (D / 4);
      float* p0 = s0 + row * RS + 4 * col;
      float* p1 = s1 + row * RS + 4 * col;
      *reinterpret_cast<f32x2*>(p0) = f32x2{r0[i][0], r0[i][1]};
      *reinterpret_cast<f32x2*>(p0 + 2) = f32x2{r0[i][2], r0[i][3]};
      *reinterpret_cast<f32x2*>(p1) = f32x2{r1[i][0], r1[i][1]};
      *reinterpret_cast<f32x2*>(p1 + 2) = f32x2{r1[i][2], r1[i][3]};
    }
  }
};

// Bias of score (qi, key) in log2 units: slope |qi - key| or the tensor entry (indices
// clamped; clamped entries are masked by the caller).
template <int BM>
__device__ inline float bias2(const BwdArgs& a, const float* TB, float slope2, int qi, int key) {
  if constexpr (BM == kBiasSlope) {
    return slope2 * __builtin_fabsf((float)(qi - key));
  } else if constexpr (BM == kBiasTensor) {
    const long long r = min(qi, a.Nq - 1), c = min(key, a.Nk - 1);
    return TB[r * a.tb_si + c] * kLog2e;
  } else {
    return 0.f;
  }
}

// ---------------------------------------------------------------------------------
// dK, dV: key-block-outer. Workgroup = 4 waves x 32 keys; 32-row query tiles of Q, dO,
// LSE*log2(e), D and the rows' key intervals through two LDS stages (register-staged).
// ---------------------------------------------------------------------------------
template <int D, int BM>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dkdv32_kernel(const BwdArgs a) {
  constexpr bool SLOPE = BM == kBiasSlope, TENSOR = BM == kBiasTensor;
  constexpr int BR = 32, RS = D + 2, NS = D / 2, DB = D / 32;
  constexpr int TILE = BR * RS, STAGE = 2 * TILE + 4 * BR;
  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];
  __shared__ int win[2];

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id(), n = lane & 31, h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const bool causal = a.causal != 0, ranged = a.key_start != nullptr;
  // dbias summed over batches and/or heads: the workgroup owns one dbias slice (slot) and
  // computes, one after the other, every (b, h) that shares it (its members), adding each
  // member's dS in a fixed order; otherwise a slot is one (b, h)
  const int rb = TENSOR ? (a.db_red & FA_DBIAS_SUM_BATCH) : 0;
  const int rh = TENSOR ? (a.db_red & FA_DBIAS_SUM_HEADS) : 0;
  const bool rrows = TENSOR && (a.db_red & FA_DBIAS_SUM_ROWS) != 0;
  const int slot_h = rh ? 1 : a.H;
  const int n_slots = (rb ? 1 : a.B) * slot_h;
  const int mem_h = rh ? a.H : 1, n_mem = (rb ? a.B : 1) * mem_h;
  int slot, kb;
  map_block(blockIdx.x, n_slots, a.nblk, a.sched, false, slot, kb);
  // the slot's dbias [Nq' rows][Nk] (NULL: dbias not wanted); dense and summed forms are
  // cleared by the launch, so every member adds (rows summed: written once at the end)
  float* dB = (TENSOR && a.dbias != nullptr) ? a.dbias + (size_t)slot * (rrows ? 1 : Nq) * Nk
                                             : nullptr;
  float dbr = 0.f;  // rows summed: this lane's share of its key's dbias, over all members

  for (int m = 0; m < n_mem; ++m) {
    if (m > 0) __syncthreads();  // every wave is done with the stages and the window
    const int bh = (rb | rh) ? (rb ? m / mem_h : slot / slot_h) * a.H
                                   + (rh ? m % mem_h : slot % slot_h)
                             : slot;
    const int head = bh % a.H;
    const float* Q = static_cast<const float*>(a.q) + (size_t)bh * Nq * D;
    const float* K = static_cast<const float*>(a.k) + (size_t)bh * Nk * D;
    const float* V = static_cast<const float*>(a.v) + (size_t)bh * Nk * D;
    const float* dO = static_cast<const float*>(a.dout) + (size_t)bh * Nq * D;
    const float* lse2 = a.lse2 + (size_t)bh * Nq;
    const float* dlt = a.delta + (size_t)bh * Nq;
    const float sl2 = a.sl2;
    const float slope2 = SLOPE ? a.slope2[a.n_slopes == 1 ? 0 : head] : 0.f;
    const float* TB = TENSOR ? a.tbias + (long long)(bh / a.H) * a.tb_sb
                                   + (long long)head * a.tb_sh
                             : nullptr;

    const int k0 = kb * 128, k1 = min(k0 + 128, Nk);
    const int kw0 = k0 + 32 * wid, kw1 = min(kw0 + 32, Nk);
    const int key = kw0 + n;

    // K and V of this lane's key: B operands of S = Q K^T and dP = dO V^T (element 2s + h)
    float kf[NS], vf[NS];
    {
      const size_t r = (size_t)min(key, Nk - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kf[s] = K[r * D + 2 * s + h];
        vf[s] = V[r * D + 2 * s + h];
      }
    }

    // query tiles that can see a key of this block (range summaries are per 64 rows)
    const int nqt = (Nq + BR - 1) / BR;
    int t_lo = 0, t_hi = nqt;
    if (causal) t_lo = max(0, k0 - off) / BR;
    if (causal && k0 - off >= Nq) t_hi = 0;
    if (ranged) {
      if (tid < 64) {
        int lo = nqt, hi = -1;
        for (int t = lane; t < nqt; t += 64) {
          const int* sm = a.qsum + 4 * (t / 2);  // {min start, max start, min end, max end}
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

    Tile32<D, RS> tl;
    float areg = 0.f;  // threads 0-127: one entry of the tile's row arrays
    auto load = [&](int t) {
      const int q0t = t * BR;
      tl.load(Q, dO, q0t, Nq, tid);
      if (tid < 4 * BR) {
        const int arr = tid / BR, r = min(q0t + tid % BR, Nq - 1);
        if (arr == 0) areg = lse2[r];
        else if (arr == 1) areg = dlt[r];
        else if (ranged) areg = __builtin_bit_cast(float, arr == 2 ? a.key_start[r] : a.key_end[r]);
      }
    };
    auto store = [&](int stg) {
      float* sb = smem + stg * STAGE;
      tl.store(sb, sb + TILE, tid);
      if (tid < 4 * BR) sb[2 * TILE + tid] = areg;
    };

    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dv[db] = f32x16{}; dk[db] = f32x16{}; }
    float sgrad = 0.f;

    if (t_lo < t_hi) {
      load(t_lo);
      store(0);
    }
    __syncthreads();
    for (int t = t_lo; t < t_hi; ++t) {
      const int stg = (t - t_lo) & 1;
      const bool more = t + 1 < t_hi;
      if (more) load(t + 1);
      sync_check();
      const int q0t = t * BR;
      const float* Qs = smem + stg * STAGE;
      const float* Ds = Qs + TILE;
      const float* Ar = Qs + 2 * TILE;  // LSE*log2(e), D, key_start, key_end (32 each)

      bool skip = kw0 >= Nk;
      if (causal) skip |= q0t + BR - 1 + off < kw0;
      if (ranged) {
        const int* sm = a.qsum + 4 * (t / 2);
        skip |= kw1 <= sm[0] || kw0 >= sm[3];
      }
      // block bitmap (a 32-row tile and a wave's 32 keys lie inside one block), as a mask
      if (a.bmask != nullptr && !skip) {
        const int bb = bh / a.H, hh = bh - bb * a.H;
        skip = a.bmask[bb * a.bm_sb + hh * a.bm_sh + (long long)(q0t / a.bq) * a.nkb +
                       min(kw0, Nk - 1) / a.bk] == 0;
      }
      if (!skip) {
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          sc = mma32(Qs[n * RS + 2 * s + h], kf[s], sc);
          dp = mma32(Ds[n * RS + 2 * s + h], vf[s], dp);
        }
        float p[16], ds[16];
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          const int r = res_row(g, h), qi = q0t + r;
          const float x = __builtin_fmaf(sc[g], sl2, bias2<BM>(a, TB, slope2, qi, key) - Ar[r]);
          bool vis = key < Nk && qi < Nq && (!causal || key <= qi + off);
          if (ranged) {
            const int lo = min(max(__builtin_bit_cast(int, Ar[2 * BR + r]), 0), Nk);
            const int hi = min(max(__builtin_bit_cast(int, Ar[3 * BR + r]), 0), Nk);
            vis = vis && key >= lo && key < hi;
          }
          p[g] = vis ? fast_exp2(x) : 0.f;
          ds[g] = p[g] * (dp[g] - Ar[BR + r]);
          if constexpr (TENSOR) {
            if (dB != nullptr && key < Nk && qi < Nq) {
              if (rrows) dbr += ds[g];
              else if (n_mem > 1) dB[(size_t)qi * Nk + key] += ds[g];
              else dB[(size_t)qi * Nk + key] = ds[g];
            }
          }
          if constexpr (SLOPE)
            sgrad = __builtin_fmaf(ds[g], __builtin_fabsf((float)(qi - key)), sgrad);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const int r = res_row(g, h);
            dv[db] = mma32(p[g], Ds[r * RS + 32 * db + n], dv[db]);
            dk[db] = mma32(ds[g], Qs[r * RS + 32 * db + n], dk[db]);
          }
        }
      }
      // the other stage was last read before the previous barrier
      if (more) store(stg ^ 1);
      __syncthreads();
    }

    if constexpr (SLOPE) {
      if (a.dslope_part != nullptr) {
        __shared__ float sred[4];
        const float w = wave_fsum(sgrad);
        if (lane == 0) sred[wid] = w;
        __syncthreads();
        if (tid == 0)
          a.dslope_part[(size_t)bh * a.nblk + kb] = sred[0] + sred[1] + sred[2] + sred[3];
      }
    }

    const float scale = a.scale;
    float* dK = static_cast<float*>(a.dk);
    float* dV = static_cast<float*>(a.dv);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int kr = kw0 + res_row(g, h);
        if (kr < Nk) {
          const size_t idx = ((size_t)bh * Nk + kr) * D + 32 * db + n;
          dK[idx] = dk[db][g] * scale;
          dV[idx] = dv[db][g];
        }
      }
    }
  }  // members
  // rows summed: the two lanes of a key hold the sums of alternate row groups
  if constexpr (TENSOR) {
    if (rrows && dB != nullptr) {
      const float tot = dbr + __shfl_xor(dbr, 32, 64);
      const int key = kb * 128 + 32 * wid + n;
      if (h == 0 && key < Nk) dB[key] = tot;
    }
  }
}

// ---------------------------------------------------------------------------------
// dQ: query-block-outer. Workgroup = 4 waves x 32 queries (lane = query); 32-key tiles of
// K and V through two LDS stages. S^T = K Q^T and dP^T = V dO^T put the key on the
// registers, so dS^T is the B operand of dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------------
template <int D, int BM>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dq32_kernel(const BwdArgs a) {
  constexpr int BC = 32, RS = D + 2, NS = D / 2, DB = D / 32;
  constexpr int TILE = BC * RS, STAGE = 2 * TILE;
  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];
  __shared__ int wg_win[4][2];

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id(), n = lane & 31, h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const bool causal = a.causal != 0, ranged = a.key_start != nullptr;
  int bh, qb;
  map_block(blockIdx.x, a.B * a.H, a.nblk, a.sched, true, bh, qb);
  const int head = bh % a.H;
  const float* Q = static_cast<const float*>(a.q) + (size_t)bh * Nq * D;
  const float* K = static_cast<const float*>(a.k) + (size_t)bh * Nk * D;
  const float* V = static_cast<const float*>(a.v) + (size_t)bh * Nk * D;
  const float* dO = static_cast<const float*>(a.dout) + (size_t)bh * Nq * D;
  const float sl2 = a.sl2;
  const float slope2 = BM == kBiasSlope ? a.slope2[a.n_slopes == 1 ? 0 : head] : 0.f;
  const float* TB = BM == kBiasTensor
                        ? a.tbias + (long long)(bh / a.H) * a.tb_sb + (long long)head * a.tb_sh
                        : nullptr;

  const int wq0 = qb * 128 + 32 * wid, qrow = wq0 + n;
  const size_t qr = (size_t)min(qrow, Nq - 1);
  float qf[NS], dof[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = Q[qr * D + 2 * s + h];
    dof[s] = dO[qr * D + 2 * s + h];
  }
  const float lq = lse_offset2(a.lse[(size_t)bh * Nq + qr]);
  const float dd = a.delta[(size_t)bh * Nq + qr];

  // this row's key interval; the wave's and the workgroup's key windows
  int kst = 0, ken = Nk;
  int w_min_s = Nk, w_max_e = 0;
  if (ranged) {
    if (qrow < Nq) {
      kst = min(max(a.key_start[qrow], 0), Nk);
      ken = min(max(a.key_end[qrow], 0), Nk);
    }
    w_min_s = wave_min(qrow < Nq ? kst : Nk);
    w_max_e = wave_max(qrow < Nq ? ken : 0);
  }
  const int wq_last = min(wq0 + 32, Nq) - 1;
  int w_lo = 0, w_hi = Nk;
  if (causal) w_hi = min(w_hi, wq_last + off + 1);
  if (ranged) {
    w_lo = max(w_lo, w_min_s);
    w_hi = min(w_hi, w_max_e);
  }
  if (wq0 >= Nq || w_hi <= w_lo) { w_lo = Nk; w_hi = 0; }
  if (lane == 0) { wg_win[wid][0] = w_lo; wg_win[wid][1] = w_hi; }
  __syncthreads();
  int g_lo = Nk, g_hi = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) { g_lo = min(g_lo, wg_win[w][0]); g_hi = max(g_hi, wg_win[w][1]); }
  const int t_lo = g_hi > g_lo ? g_lo / BC : 0;
  const int t_hi = g_hi > g_lo ? (g_hi + BC - 1) / BC : 0;

  Tile32<D, RS> tl;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  if (t_lo < t_hi) {
    tl.load(K, V, t_lo * BC, Nk, tid);
    tl.store(smem, smem + TILE, tid);
  }
  __syncthreads();
  for (int t = t_lo; t < t_hi; ++t) {
    const int stg = (t - t_lo) & 1;
    const bool more = t + 1 < t_hi;
    if (more) tl.load(K, V, (t + 1) * BC, Nk, tid);
    sync_check();
    const int kt0 = t * BC;
    const float* Ks = smem + stg * STAGE;
    const float* Vs = Ks + TILE;
    // block bitmap: this lane's row and the tile's 32 keys lie inside one block
    bool blk = true;
    if (a.bmask != nullptr) {
      const int bb = bh / a.H, hh = bh - bb * a.H;
      blk = a.bmask[bb * a.bm_sb + hh * a.bm_sh + (long long)((int)qr / a.bq) * a.nkb +
                    min(kt0, Nk - 1) / a.bk] != 0;
    }
    if (!(kt0 >= w_hi || kt0 + BC <= w_lo)) {
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        st = mma32(Ks[n * RS + 2 * s + h], qf[s], st);
        dpt = mma32(Vs[n * RS + 2 * s + h], dof[s], dpt);
      }
      float ds[16];
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const int key = kt0 + res_row(g, h);
        const float x = __builtin_fmaf(st[g], sl2, bias2<BM>(a, TB, slope2, qrow, key) - lq);
        const bool vis = blk && key < Nk && qrow < Nq && (!causal || key <= qrow + off) &&
                         key >= kst && key < ken;
        const float p = vis ? fast_exp2(x) : 0.f;
        ds[g] = p * (dpt[g] - dd);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 16; ++g)
          acc[db] = mma32(Ks[res_row(g, h) * RS + 32 * db + n], ds[g], acc[db]);
      }
    }
    if (more) tl.store(smem + (stg ^ 1) * STAGE, smem + (stg ^ 1) * STAGE + TILE, tid);
    __syncthreads();
  }

  // lane holds dQ^T[32 db + res_row(g, h)][query qrow]
  if (qrow < Nq) {
    const float scale = a.scale;
    float* dQ = static_cast<float*>(a.dq) + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 16; ++g) dQ[32 * db + res_row(g, h)] = acc[db][g] * scale;
    }
  }
}

// Clears n floats (dbias before the dK/dV pass writes the visible entries; a kernel
// rather than a memset node, so that a captured graph replays it correctly).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0.f;
}

template <int D, int BM>
hipError_t launch_passes(int phases, BwdArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  hipError_t e = hipSuccess;
  const int sched = (BH % 8 == 0) ? 1 : 0;
  if (phases & FA_BWD_DKDV) {
    BwdArgs b = a;
    b.nblk = (a.Nk + 127) / 128;
    // a workgroup per dbias slice and key block (a slice is one (b, h) unless dbias is
    // summed over batches or heads)
    int slots = BH;
    if (BM == kBiasTensor && a.dbias != nullptr) {
      slots = ((a.db_red & FA_DBIAS_SUM_BATCH) ? 1 : a.B) *
              ((a.db_red & FA_DBIAS_SUM_HEADS) ? 1 : a.H);
      if ((a.db_red & FA_DBIAS_SUM_ROWS) == 0) {  // rows summed: every element is written
        const size_t nd = (size_t)slots * a.Nq * a.Nk;
        const unsigned zb = (unsigned)std::min<size_t>((nd + 255) / 256, 8192);
        hipLaunchKernelGGL(zero_f32_kernel, dim3(zb), dim3(256), 0, st, a.dbias, nd);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    } else {
      b.db_red = 0;
    }
    b.sched = (slots % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((dkdv32_kernel<D, BM>), dim3((unsigned)(slots * b.nblk)), dim3(256), 0, st,
                       b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (BM == kBiasSlope && a.dslopes != nullptr) {
      e = launch_dslope_reduce(b.dslope_part, a.B, a.H, b.nblk, a.n_slopes, a.dslopes, st);
      if (e != hipSuccess) return e;
    }
  }
  if (phases & FA_BWD_DQ) {
    BwdArgs b = a;
    b.nblk = (a.Nq + 127) / 128;
    b.sched = sched;
    hipLaunchKernelGGL((dq32_kernel<D, BM>), dim3((unsigned)(BH * b.nblk)), dim3(256), 0, st, b);
    e = hipGetLastError();
  }
  return e;
}

template <int D>
hipError_t launch_d(int bias, int phases, BwdArgs& a, hipStream_t st) {
  if (phases & FA_BWD_PREP) {
    const int rows = a.B * a.H * a.Nq;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((prep32_kernel<D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, st,
                       static_cast<const float*>(a.o), static_cast<const float*>(a.dout), a.lse,
                       a.delta, a.lse2, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.key_start != nullptr) {
      e = launch_mask_summary(a.key_start, a.key_end, a.Nq, a.Nk, kDkdvBR, a.qsum, st);
      if (e != hipSuccess) return e;
    }
  }
  if (bias == kBiasTensor) return launch_passes<D, kBiasTensor>(phases, a, st);
  if (bias == kBiasSlope) return launch_passes<D, kBiasSlope>(phases, a, st);
  return launch_passes<D, kBiasNone>(phases, a, st);
}

}  // namespace

hipError_t launch_bwd32(int d, int bias, int phases, BwdArgs& a, hipStream_t st) {
  return d == 128 ? launch_d<128>(bias, phases, a, st) : launch_d<64>(bias, phases, a, st);
}

}  // namespace fa
