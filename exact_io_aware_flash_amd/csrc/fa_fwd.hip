// fa_fwd.hip -- fused exact-attention forward kernel for gfx950 (MI355X).
//
// Method (blog "Apakah Konteks Sehari Penuh Mengalahkan Konteks Sepuluh Menit?",
// sections "Algoritma Flash Attention", "Pengulangan softmax online", "FA2: paralelisme",
// "Causal masking ..."): Q is cut into row blocks and K/V into column blocks; for every
// query block the kernel walks the key/value blocks, computes the score tile on chip,
// keeps a running row max and row sum, rescales the output accumulator when the max
// grows, and divides by the row sum once at the end. Tiles that hold no visible key are
// never loaded or computed. The score matrix never leaves registers.
//
// gfx950 mapping (not the Hopper design the pages describe):
//  * one workgroup = NW waves x 32 query rows of one (batch, head); the grid runs over
//    (batch, head, query block[, key range]) so batch 1-4 still fills 256 CUs;
//  * each wave owns its own 32 query rows (no cross-wave reduction of scores);
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}:
//    a lane then holds 16 keys of ONE query row per 32x32 tile, so the row statistics
//    are per lane except for one exchange between the two wave halves;
//  * the probabilities feed O^T += V^T P^T directly from those result registers; V stays
//    row-major in LDS and its transposed operand comes from ds_read_b64_tr_b16;
//  * K and V tiles go from HBM straight into a ring of LDS stages (buffer loads that
//    write LDS), one or more tiles ahead of the tile being computed, one barrier a tile;
//  * the running max is only moved when a row's scores exceed it by more than 2^8
//    (exact: numerator and denominator share the same stale max); once every row holds
//    a finite max, a tile's own max is not even computed: a score above m + 8 makes the
//    lane's probability sum exceed 2^8, and only then is the max taken and the tile redone;
//  * the exponents (scaled score + bias - running max) are formed in place right after
//    the score products, so the probability pass is exp2, sum and packing only;
//  * Q stays in registers for the whole loop; O^T and S^T live in registers.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

template <typename T, int D_, int BC_, int QSUB_, int NW_>
struct FwdCfg {
  static constexpr bool kF32 = std::is_same<T, float>::value;
  static constexpr int D = D_, BC = BC_, QSUB = QSUB_, NW = NW_;
  static constexpr int kNT = NW * 64;
  static constexpr int kQW = 32 * QSUB;       // query rows per wave
  static constexpr int kBR = kQW * NW;        // query rows per workgroup
  static constexpr int kKB = BC / 32;         // 32-key blocks per tile
  static constexpr int kDB = D / 32;          // 32-wide d blocks of O^T
  static constexpr int kDK = kF32 ? D / 2 : D / 16;  // MFMA k-steps over d for S^T
  // LDS layout. 16-bit: K row-major (row stride D*2+16 bytes), V^T rows of BC keys
  // (stride BC*2+16, 16-byte chunks XOR-swizzled by (row/16)). f32: K row stride
  // (D+1)*4 (odd word stride), V row-major with stride (D+4)*4.
  static constexpr int kKStride = kF32 ? (D + 1) * 4 : D * 2 + 16;
  static constexpr int kVStride = kF32 ? (D + 4) * 4 : BC * 2 + 16;
  static constexpr int kKBytes = align16(BC * kKStride);
  static constexpr int kVBytes = kF32 ? BC * kVStride : D * kVStride;
  static constexpr int kStage = kKBytes + kVBytes;
  // global->LDS copy split: 16-byte chunks per thread
  static constexpr int kEltPerChunk = kF32 ? 4 : 8;
  static constexpr int kRowChunks = D / kEltPerChunk;
  static constexpr int kKPer = BC * kRowChunks / kNT;
  // 16-bit V: a thread owns KQ consecutive keys x 8 d values (one chunk per key)
  static constexpr int kKQraw = BC * kRowChunks / kNT;
  static constexpr int kKQ = kF32 ? 1 : (kKQraw >= 4 ? 4 : kKQraw);
  static constexpr int kVPer = kF32 ? kKPer : BC * kRowChunks / (kKQ * kNT);
  static constexpr int kVChunksSwz = BC / 8;   // 16-byte chunks per V^T row
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(kKPer >= 1 && kKPer * kNT == BC * kRowChunks, "K copy split");
  static_assert(kF32 || (kKQ >= 2 && kVPer * kKQ * kNT == BC * kRowChunks), "V copy split");
  static_assert(2 * kStage <= 160 * 1024, "LDS budget");
};

// Keys inside a tile are relabelled in V^T so that the 8 keys one lane feeds to a
// P.V MFMA step are contiguous: swap bits 2 and 3 of the tile-local key index.
__device__ constexpr int vt_pos(int key) { return tr_pos(key); }

template <class C>
__device__ inline int vt_off(int row, int chunk) {
  return row * C::kVStride + 16 * (chunk ^ ((row >> 4) & (C::kVChunksSwz - 1)));
}

template <typename T, int D, int BC, int QSUB, int NW, int WPE, int BM>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(const FwdArgs a) {
  using C = FwdCfg<T, D, BC, QSUB, NW>;
  using E = Elt<T>;
  constexpr bool F32 = C::kF32;
  constexpr bool SLOPE = BM == kBiasSlope, TENSOR = BM == kBiasTensor;
  constexpr bool PRE = BM != kBiasNone;  // scores scaled to log2 units before the row max
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kStage];
  __shared__ int wg_win[NW][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk;
  const int off = Nk - Nq;  // bottom-right aligned causal diagonal
  const bool causal = a.causal != 0;
  const bool ranged = a.key_start != nullptr;

  // work unit = (b, h, query block, key range); heaviest query blocks first
  int bh, unit;
  map_block(blockIdx.x, a.B * a.H, a.nqb * a.n_split, a.sched, true, bh, unit);
  const int qb = unit / a.n_split, split = unit - qb * a.n_split;
  const int head = bh % a.H;
  const int q0 = qb * C::kBR;
  const T* __restrict__ Q = static_cast<const T*>(a.q) + (size_t)bh * Nq * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + (size_t)bh * Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + (size_t)bh * Nk * D;
  T* __restrict__ O = static_cast<T*>(a.o) + (size_t)bh * Nq * D;
  const float sl2 = a.sl2;
  const float slope2 = SLOPE ? a.slope2[a.n_slopes == 1 ? 0 : head] : 0.f;
  const float* TB = TENSOR ? a.tbias + (long long)(bh / a.H) * a.tb_sb + (long long)head * a.tb_sh
                           : nullptr;

  // ---- this lane's query rows and key intervals ----------------------------------
  const int wq0 = q0 + wid * C::kQW;
  int qrow[QSUB], kst[QSUB], ken[QSUB];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    qrow[qs] = wq0 + qs * 32 + n;
    kst[qs] = 0;
    ken[qs] = Nk;
    if (ranged && qrow[qs] < Nq) {
      kst[qs] = min(max(a.key_start[qrow[qs]], 0), Nk);
      ken[qs] = min(max(a.key_end[qrow[qs]], 0), Nk);
    }
  }
  // wave-uniform summaries of the rows' key intervals (rows past the end take no part);
  // per-lane partials live only inside the uniform branch, so the results stay scalar
  int w_min_s = Nk, w_max_s = 0, w_min_e = Nk, w_max_e = 0;
  if (ranged) {
    int s0 = Nk, s1 = 0, e0 = Nk, e1 = 0;
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs)
      if (qrow[qs] < Nq) {
        s0 = min(s0, kst[qs]); s1 = max(s1, kst[qs]);
        e0 = min(e0, ken[qs]); e1 = max(e1, ken[qs]);
      }
    w_min_s = wave_min(s0);
    w_max_s = wave_max(s1);
    w_min_e = wave_min(e0);
    w_max_e = wave_max(e1);
  }
  const bool wave_live = wq0 < Nq;
  const int wq_last = min(wq0 + C::kQW, Nq) - 1;
  // keys [w_lo, w_hi) may be visible to some row of this wave; keys < w_full_c are
  // visible (causally) to every row of the wave
  int w_lo = 0, w_hi = Nk, w_full_c = Nk;
  if (causal) {
    w_hi = min(w_hi, wq_last + off + 1);
    w_full_c = max(0, min(Nk, wq0 + off + 1));
  }
  if (ranged) {
    w_lo = max(w_lo, w_min_s);
    w_hi = min(w_hi, w_max_e);
  }
  if (a.n_split > 1) {  // this unit's key range (whole tiles)
    w_lo = max(w_lo, split * a.split_keys);
    w_hi = min(w_hi, (split + 1) * a.split_keys);
  }
  if (!wave_live || w_hi <= w_lo) { w_lo = Nk; w_hi = 0; }
  if (lane == 0) { wg_win[wid][0] = w_lo; wg_win[wid][1] = w_hi; }
  __syncthreads();
  int g_lo = Nk, g_hi = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { g_lo = min(g_lo, wg_win[w][0]); g_hi = max(g_hi, wg_win[w][1]); }
  const int t_lo = g_hi > g_lo ? g_lo / BC : 0;
  const int t_hi = g_hi > g_lo ? (g_hi + BC - 1) / BC : 0;

  // ---- Q fragments in registers (B operand of S^T = K Q^T) -----------------------
  u32x4 qf[QSUB][F32 ? 1 : C::kDK];
  float qf1[QSUB][F32 ? C::kDK : 1];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const size_t r = (size_t)min(qrow[qs], Nq - 1);  // rows past the end are never stored
    if constexpr (F32) {
#pragma unroll
      for (int ks = 0; ks < C::kDK; ++ks) qf1[qs][ks] = Q[r * D + 2 * ks + h];
    } else {
#pragma unroll
      for (int ks = 0; ks < C::kDK; ++ks) qf[qs][ks] = ldg16(Q + r * D + 16 * ks + 8 * h);
    }
  }

  // ---- running state ---------------------------------------------------------------
  f32x16 o[QSUB][C::kDB];
  float m2[QSUB], l[QSUB];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    m2[qs] = kNegInf;
    l[qs] = 0.f;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) o[qs][db] = f32x16{};
  }

  // ---- global -> register -> LDS copy of one K/V tile ------------------------------
  u32x4 kreg[C::kKPer];
  u32x4 vreg[C::kVPer][F32 ? 1 : C::kKQ];

  auto load_tile = [&](int t) {
    const int kt0 = t * BC;
#pragma unroll
    for (int i = 0; i < C::kKPer; ++i) {
      const int c = tid + i * C::kNT;
      const int row = c / C::kRowChunks, col = c % C::kRowChunks;
      const int key = min(kt0 + row, Nk - 1);
      kreg[i] = ldg16(K + (size_t)key * D + col * C::kEltPerChunk);
    }
    if constexpr (F32) {
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int c = tid + i * C::kNT;
        const int row = c / C::kRowChunks, col = c % C::kRowChunks;
        const int key = min(kt0 + row, Nk - 1);
        vreg[i][0] = ldg16(V + (size_t)key * D + col * 4);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int b = tid + i * C::kNT;
        const int grp = b / C::kRowChunks, col = b % C::kRowChunks;
#pragma unroll
        for (int e = 0; e < C::kKQ; ++e) {
          const int key = min(kt0 + grp * C::kKQ + e, Nk - 1);
          vreg[i][e] = ldg16(V + (size_t)key * D + col * 8);
        }
      }
    }
  };

  auto store_tile = [&](int stage) {
    char* Ks = smem + stage * C::kStage;
    char* Vs = Ks + C::kKBytes;
    if constexpr (F32) {
#pragma unroll
      for (int i = 0; i < C::kKPer; ++i) {
        const int c = tid + i * C::kNT;
        const int row = c / C::kRowChunks, col = c % C::kRowChunks;
#pragma unroll
        for (int e = 0; e < 4; ++e) lds_st4(Ks, row * C::kKStride + (col * 4 + e) * 4, kreg[i][e]);
      }
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int c = tid + i * C::kNT;
        const int row = c / C::kRowChunks, col = c % C::kRowChunks;
        lds_st16(Vs, row * C::kVStride + col * 16, vreg[i][0]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::kKPer; ++i) {
        const int c = tid + i * C::kNT;
        const int row = c / C::kRowChunks, col = c % C::kRowChunks;
        lds_st16(Ks, row * C::kKStride + col * 16, kreg[i]);
      }
      // V^T: the thread holds keys grp*KQ .. +KQ-1, d values col*8 .. col*8+7
#pragma unroll
      for (int i = 0; i < C::kVPer; ++i) {
        const int b = tid + i * C::kNT;
        const int grp = b / C::kRowChunks, col = b % C::kRowChunks;
        const int pos = vt_pos(grp * C::kKQ);  // KQ consecutive keys -> KQ consecutive slots
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int row = col * 8 + dd;
          const int w = dd >> 1;
          const int byte = vt_off<C>(row, pos >> 3) + (pos & 7) * 2;
          if constexpr (C::kKQ == 4) {
            u32x2 val;
            val[0] = (dd & 1) ? pack_hi(vreg[i][0][w], vreg[i][1][w]) : pack_lo(vreg[i][0][w], vreg[i][1][w]);
            val[1] = (dd & 1) ? pack_hi(vreg[i][2][w], vreg[i][3][w]) : pack_lo(vreg[i][2][w], vreg[i][3][w]);
            lds_st8(Vs, byte, val);
          } else {
            const uint32_t val = (dd & 1) ? pack_hi(vreg[i][0][w], vreg[i][1][w]) : pack_lo(vreg[i][0][w], vreg[i][1][w]);
            lds_st4(Vs, byte, val);
          }
        }
      }
    }
  };

  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int stage = (t - t_lo) & 1;
    const bool more = t + 1 < t_hi;
    if (more) load_tile(t + 1);
    sync_check();

    const int kt0 = t * BC;
    const int kt1 = kt0 + BC;
    const bool skip = kt0 >= w_hi || kt1 <= w_lo;
    if (!skip) {
      const bool full = a.bmask == nullptr && kt1 <= Nk && kt1 <= w_full_c &&
                        (!ranged || (w_max_s <= kt0 && w_min_e >= kt1));
      const char* Ks = smem + stage * C::kStage;
      const char* Vs = Ks + C::kKBytes;

      // ---- S^T = K Q^T ---------------------------------------------------------
      f32x16 s[QSUB][C::kKB];
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb) s[qs][kb] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb) {
#pragma unroll
        for (int ks = 0; ks < C::kDK; ++ks) {
          if constexpr (F32) {
            const float av = *reinterpret_cast<const float*>(
                Ks + (kb * 32 + n) * C::kKStride + (2 * ks + h) * 4);
#pragma unroll
            for (int qs = 0; qs < QSUB; ++qs) s[qs][kb] = E::mma1(av, qf1[qs][ks], s[qs][kb]);
          } else {
            const u32x4 av = lds_ld16(Ks, (kb * 32 + n) * C::kKStride + 32 * ks + 16 * h);
#pragma unroll
            for (int qs = 0; qs < QSUB; ++qs) s[qs][kb] = E::mma(av, qf[qs][ks], s[qs][kb]);
          }
        }
      }

      // ---- bias and masking (masking only on partially visible tiles) ----------
      if constexpr (TENSOR) {
        // the bias entries of this lane's row and keys, read straight from memory (this
        // kernel stages K and V through registers, so plain loads need no extra wait);
        // indices clamped into the matrix, clamped entries are masked below
#pragma unroll
        for (int qs = 0; qs < QSUB; ++qs) {
          const float* brow = TB + (long long)min(qrow[qs], Nq - 1) * a.tb_si;
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
            for (int g = 0; g < 16; ++g) {
              const int j = min(kt0 + kb * 32 + res_row(g, h), Nk - 1);
              s[qs][kb][g] = __builtin_fmaf(s[qs][kb][g], sl2, brow[j] * kLog2e);
            }
        }
      }
      if constexpr (SLOPE) {
#pragma unroll
        for (int qs = 0; qs < QSUB; ++qs) {
          const float base = (float)(qrow[qs] - kt0 - 4 * h);
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
            for (int g = 0; g < 16; ++g) {
              const float dist = base - (float)(kb * 32 + 8 * (g / 4) + (g % 4));
              s[qs][kb][g] = __builtin_fmaf(s[qs][kb][g], sl2, slope2 * __builtin_fabsf(dist));
            }
        }
      }
      if (!full) {
#pragma unroll
        for (int qs = 0; qs < QSUB; ++qs) {
          const int lo = kst[qs], hi = min(ken[qs], Nk);
          const int cl = causal ? qrow[qs] + off : Nk;
#pragma unroll
          for (int kb = 0; kb < C::kKB; ++kb) {
            // block bitmap: the 32 keys of a block lie inside one block of >= 64 keys;
            // applied here as a mask (these tiles are still loaded)
            bool blk = true;
            if (a.bmask != nullptr) {
              const int bb = bh / a.H, hh = bh - bb * a.H;
              const int r = min(qrow[qs], Nq - 1) / a.bq;
              const int c = min(kt0 + kb * 32, Nk - 1) / a.bk;
              blk = a.bmask[bb * a.bm_sb + hh * a.bm_sh + (long long)r * a.nkb + c] != 0;
            }
#pragma unroll
            for (int g = 0; g < 16; ++g) {
              const int j = kt0 + kb * 32 + res_row(g, h);
              const bool vis = blk && j >= lo && j < hi && j <= cl;
              s[qs][kb][g] = vis ? s[qs][kb][g] : kNegInf;
            }
          }
        }
      }

      // ---- online softmax: tile row max, lazy rescale, exponentials, row sums -----
      float tmax[QSUB];
      bool need = false;
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
          for (int g = 0; g < 16; ++g) mx = __builtin_fmaxf(mx, s[qs][kb][g]);
        mx = __builtin_fmaxf(mx, xhalf(mx));
        tmax[qs] = PRE ? mx : mx * sl2;
        need |= tmax[qs] > m2[qs] + kTau;
      }
      if (wave_any(need)) {
#pragma unroll
        for (int qs = 0; qs < QSUB; ++qs) {
          const float mnew = __builtin_fmaxf(m2[qs], tmax[qs]);
          const float alpha = mnew == kNegInf ? 1.f : fast_exp2(m2[qs] - mnew);
          l[qs] *= alpha;
#pragma unroll
          for (int db = 0; db < C::kDB; ++db) o[qs][db] *= alpha;
          m2[qs] = mnew;
        }
      }
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs) {
        const float nb = m2[qs] == kNegInf ? 0.f : -m2[qs];
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::kKB; ++kb)
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const float x = PRE ? s[qs][kb][g] + nb : __builtin_fmaf(s[qs][kb][g], sl2, nb);
            const float p = fast_exp2(x);
            s[qs][kb][g] = p;
            rs += p;
          }
        l[qs] += rs;
      }

      // ---- O^T += V^T P^T ---------------------------------------------------------
#pragma unroll
      for (int kb = 0; kb < C::kKB; ++kb) {
        if constexpr (F32) {
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const int key = kb * 32 + res_row(g, h);
#pragma unroll
            for (int db = 0; db < C::kDB; ++db) {
              const float av = *reinterpret_cast<const float*>(
                  Vs + key * C::kVStride + (db * 32 + n) * 4);
#pragma unroll
              for (int qs = 0; qs < QSUB; ++qs) o[qs][db] = E::mma1(av, s[qs][kb][g], o[qs][db]);
            }
          }
        } else {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            u32x4 pb[QSUB];
#pragma unroll
            for (int qs = 0; qs < QSUB; ++qs) {
#pragma unroll
              for (int w = 0; w < 4; ++w)
                pb[qs][w] = E::pack2(s[qs][kb][8 * st + 2 * w], s[qs][kb][8 * st + 2 * w + 1]);
            }
#pragma unroll
            for (int db = 0; db < C::kDB; ++db) {
              const u32x4 av = lds_ld16(Vs, vt_off<C>(db * 32 + n, 4 * kb + 2 * st + h));
#pragma unroll
              for (int qs = 0; qs < QSUB; ++qs) o[qs][db] = E::mma(av, pb[qs], o[qs][db]);
            }
          }
        }
      }
    }

    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 -------------------------------
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const float lt = l[qs] + xhalf(l[qs]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int row = qrow[qs];
    if (row < Nq && a.n_split > 1) {
      // normalised float32 partial of this key range and its LSE (nothing visible in the
      // range: O = 0, LSE = -inf, which gives it zero weight in the merge)
      const size_t prow = (size_t)split * ((size_t)a.B * a.H * Nq) + (size_t)bh * Nq + row;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * h;
          *reinterpret_cast<f32x4*>(a.o_part + prow * D + d0) =
              f32x4{o[qs][db][4 * g4] * inv, o[qs][db][4 * g4 + 1] * inv,
                    o[qs][db][4 * g4 + 2] * inv, o[qs][db][4 * g4 + 3] * inv};
        }
      if (h == 0)
        a.lse_part[prow] = lt > 0.f ? (m2[qs] + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
    } else if (row < Nq) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * h;
          const float v0 = o[qs][db][4 * g4 + 0] * inv, v1 = o[qs][db][4 * g4 + 1] * inv;
          const float v2 = o[qs][db][4 * g4 + 2] * inv, v3 = o[qs][db][4 * g4 + 3] * inv;
          if constexpr (F32) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(O) + (size_t)row * D + d0) =
                f32x4{v0, v1, v2, v3};
          } else {
            stg8(O + (size_t)row * D + d0, u32x2{E::pack2(v0, v1), E::pack2(v2, v3)});
          }
        }
      }
      if (h == 0 && a.lse != nullptr) {
        const float lse = lt > 0.f ? (m2[qs] + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
        a.lse[(size_t)bh * Nq + row] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// 16-bit forward. K and V tiles are copied straight from HBM into a ring of LDS stages by
// direct loads (no staging registers), ST - 1 tiles ahead of the one being
// computed; one barrier per tile. Tiles are swizzled (see DmaTile): K rows feed the A
// operand of S^T = K Q^T with 16-byte reads, V is gathered with transposing reads for
// the A operand of O^T = V^T P^T.
// ---------------------------------------------------------------------------------
template <int D_, int BC_, int NW_, int ST_>
struct Fwd16Cfg {
  static constexpr int D = D_, BC = BC_, NW = NW_;
  static constexpr int kNT = NW * 64;
  static constexpr int kBR = 32 * NW;       // query rows per workgroup
  static constexpr int kKB = BC / 32;       // 32-key blocks per tile
  static constexpr int kDB = D / 32;        // 32-wide d blocks of O^T
  static constexpr int kDK = D / 16;        // k-steps over d for S^T
  static constexpr int kRB = 2 * D;         // bytes per tile row
  static constexpr int kST = ST_;            // LDS ring stages (ST-1 tiles in flight)
  using Tile = DmaTile<BC, D, NW>;
  static constexpr int kStage = 2 * Tile::kBytes;  // K tile, then V tile
  static_assert(kST >= 2 && kST * kStage <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int BC, int NW, int ST, int BM, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(2, 2)))
void fwd16_kernel(const FwdArgs a) {
  using C = Fwd16Cfg<D, BC, NW, ST>;
  using E = Elt<T>;
  using BT = BiasRowTile<BC>;
  constexpr bool SLOPE = BM == kBiasSlope, TENSOR = BM == kBiasTensor;
  constexpr int KB = C::kKB, DB = C::kDB, DK = C::kDK, RB = C::kRB;
  constexpr int P = ST - 1;                                  // tiles in flight ahead
  // direct loads per wave per tile: K and V windows (+ the bias tile's rows)
  constexpr int kOpsPerTile = 2 * C::Tile::kOpsPerWave + (TENSOR ? BT::kOps : 0);
  // a stage: K tile, V tile (+ each wave's bias rows)
  constexpr int kStage = C::kStage + (TENSOR ? NW * BT::kWaveBytes : 0);
  static_assert(!TENSOR || ST == 2, "bias tensor: one tile in flight");
  static_assert(ST * kStage <= 160 * 1024, "LDS budget");
  // One LDS array per ring stage, and a loop unrolled over the stages so that every
  // access names its array: the compiler can then tell the stage being read from the
  // stages the direct loads are filling, and adds no wait on those loads.
  static_assert(ST >= 2 && ST <= 4, "two to four ring stages");
  __shared__ __attribute__((aligned(1024))) char stg0[kStage];
  __shared__ __attribute__((aligned(1024))) char stg1[kStage];
  __shared__ __attribute__((aligned(1024))) char stg2[ST > 2 ? kStage : 1];
  __shared__ __attribute__((aligned(1024))) char stg3[ST > 3 ? kStage : 1];
  __shared__ int wg_win[NW][2];
  auto sptr = [&](auto J) -> char* {
    constexpr int j = decltype(J)::value % ST;
    if constexpr (j == 0) return stg0;
    else if constexpr (j == 1) return stg1;
    else if constexpr (j == 2) return stg2;
    else return stg3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk;
  const int off = Nk - Nq;
  const bool causal = a.causal != 0;
  const bool ranged = a.key_start != nullptr;

  // work unit = (b, h, query block, key range); heaviest query blocks first
  int bh, unit;
  map_block(blockIdx.x, a.B * a.H, a.nqb * a.n_split, a.sched, true, bh, unit);
  const int qb = unit / a.n_split, split = unit - qb * a.n_split;
  const int head = bh % a.H;
  const T* __restrict__ Q = static_cast<const T*>(a.q) + (size_t)bh * Nq * D;
  const T* __restrict__ K = static_cast<const T*>(a.k) + (size_t)bh * Nk * D;
  const T* __restrict__ V = static_cast<const T*>(a.v) + (size_t)bh * Nk * D;
  T* __restrict__ O = static_cast<T*>(a.o) + (size_t)bh * Nq * D;
  const float sl2 = a.sl2;
  const float slope2 = SLOPE ? a.slope2[a.n_slopes == 1 ? 0 : head] : 0.f;
  const float* TB = TENSOR ? a.tbias + (long long)(bh / a.H) * a.tb_sb + (long long)head * a.tb_sh
                           : nullptr;

  // ---- rows, key intervals, windows -----------------------------------------------
  const int wq0 = qb * C::kBR + wid * 32;
  const int qrow = wq0 + n;
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
  if (a.n_split > 1) {  // this unit's key range (whole tiles)
    w_lo = max(w_lo, split * a.split_keys);
    w_hi = min(w_hi, (split + 1) * a.split_keys);
  }
  if (!wave_live || w_hi <= w_lo) { w_lo = Nk; w_hi = 0; }
  if (lane == 0) { wg_win[wid][0] = w_lo; wg_win[wid][1] = w_hi; }
  __syncthreads();
  int g_lo = Nk, g_hi = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { g_lo = min(g_lo, wg_win[w][0]); g_hi = max(g_hi, wg_win[w][1]); }
  const int t_lo = g_hi > g_lo ? g_lo / BC : 0;
  const int t_hi = g_hi > g_lo ? (g_hi + BC - 1) / BC : 0;
  // wave-uniform tile tests (scalar branches)
  auto live_tile = [&](int t) { return t * BC < w_hi && (t + 1) * BC > w_lo; };
  auto full_tile = [&](int t) {
    const int k0 = t * BC, k1 = k0 + BC;
    return k1 <= Nk && k1 <= w_full_c && (!ranged || (w_max_s <= k0 && w_min_e >= k1));
  };

  // ---- block-sparse bitmap: the tiles the workgroup loads ---------------------------
  // Blocks are whole tiles for every wave (block sizes are multiples of 64, tiles and
  // waves are 64 or 32 aligned), so a tile is either skipped or computed like any other.
  // Each wave marks the tiles of [t_lo, t_hi) it needs (its window and its bitmap row)
  // in 64-tile words; wave 0 compacts their union, in order, into the list the ring
  // walks, so tiles no wave needs are never loaded.
  constexpr int kMaxT = SPARSE ? kSparseMaxTiles * 32 / BC : 64;
  __shared__ uint32_t need_w[SPARSE ? NW : 1][2 * (kMaxT / 64)];  // per-wave 64-tile masks
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
      return brow != nullptr && live_tile(t) && brow[(t * BC) / a.bk] != 0;
    });
  }
  ListWindow<kMaxT> lw;
  if constexpr (SPARSE) lw.init(tlist, lane);
  // tile at ring position p, and whether this wave computes it
  auto tile_at = [&](int p) -> int {
    if constexpr (SPARSE) return (int)(lw.at(p) & 0xffffu);
    else return t_lo + p;
  };
  auto wave_needs = [&](int p, int t) -> bool {
    if constexpr (SPARSE) return (lw.at(p) >> (16 + wid)) & 1u;
    else return live_tile(t);
  };

  // ---- Q fragments (B operand of S^T = K Q^T) -------------------------------------
  u32x4 qf[DK];
  {
    const size_t r = (size_t)min(qrow, Nq - 1);  // rows past the end are never stored
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) qf[ks] = ldg16(Q + r * D + 16 * ks + 8 * h);
  }

  // ---- per-lane LDS offsets inside a swizzled tile ----------------------------------
  // K: lane n reads key row 32kb + n, d = 16ks + 8h .. +7, i.e. chunk 2ks + h.
  int ka[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) ka[ks] = n * RB + 16 * ((2 * ks + h) ^ swz<D>(n));
  // V by transposing loads: for MFMA k-slots 8h+4p .. +3 a lane needs keys
  // 32kb + 16st + 8p + 4h + {0..3} at d = 32db + n; lane 4k+q of its 16-lane group
  // addresses key row (.. + k) at columns 16*(n/16) + 4q .. +3 (chunk 4db + 2(n/16) +
  // q/2, byte 8(q&1)). kb and st move whole 16-row groups, which keep the swizzle.
  int va[DB][2];
  {
    const int q = (lane >> 2) & 3, g16 = (lane >> 4) & 1, lo2 = lane & 3;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 8 * p + 4 * h + q;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        va[db][p] = r * RB + 16 * ((4 * db + 2 * g16 + (lo2 >> 1)) ^ swz<D>(r)) + 8 * (lo2 & 1);
    }
  }
  auto vfrag = [&](const char* Vs, int db, int kb, int st) {
    const int rows = (32 * kb + 16 * st) * RB;
    const u32x2 lo = lds_ld8_tr(Vs, rows + va[db][0]);
    const u32x2 hi = lds_ld8_tr(Vs, rows + va[db][1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m2 = kNegInf, l = 0.f;

  // One key tile: S^T = K Q^T, (bias), (mask: a small branch of its own, so both outcomes
  // share the rest), running max, exponentials, O^T += V^T P^T.
  auto tile = [&](const char* Ks, const char* Vs, const char* Bs, int kt0, bool masked)
                  __attribute__((always_inline)) {
    f32x16 sc[KB];
    {
      // Every K operand of the tile is requested before the first MFMA: the scheduler
      // barrier keeps the compiler from re-interleaving the reads with the MFMAs, which
      // would leave each MFMA of the first block waiting out a full LDS latency.
      u32x4 kf[KB][DK];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) kf[kb][ks] = lds_ld16(Ks, kb * 32 * RB + ka[ks]);
      sched_fence();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) sc[kb] = E::mma(kf[kb][ks], qf[ks], sc[kb]);
      }
    }
    // The exponents, in place: x = s * scale * log2(e) + bias - m2 (m2 taken as 0 for rows
    // without a finite running max yet), formed right after the products.
    const float nb0 = m2 == kNegInf ? 0.f : -m2;
    if constexpr (SLOPE) {
      // slope2 * |i - j| with i - j = base - (kb*32 + 8*(g/4) + g%4); when every key of the
      // tile lies on one side of every row of the wave (a wave-uniform test), |i - j| is
      // +-(i - j) and bias and offset together are one multiply-add per score
      const float base = (float)(qrow - kt0 - 4 * h);
      const bool below = kt0 + BC <= wq0 + 1, above = kt0 >= wq0 + 31;
      if (below || above) {
        const float sg = below ? slope2 : -slope2, a = __builtin_fmaf(sg, base, nb0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int g = 0; g < 16; ++g)
            sc[kb][g] = __builtin_fmaf(sc[kb][g], sl2,
                                       __builtin_fmaf(-sg, (float)(kb * 32 + 8 * (g / 4) + (g % 4)), a));
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const float dist = base - (float)(kb * 32 + 8 * (g / 4) + (g % 4));
            sc[kb][g] = __builtin_fmaf(sc[kb][g], sl2, __builtin_fmaf(slope2, __builtin_fabsf(dist), nb0));
          }
      }
    } else if constexpr (!TENSOR) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int g = 0; g < 16; ++g) sc[kb][g] = __builtin_fmaf(sc[kb][g], sl2, nb0);
    }
    if constexpr (TENSOR) {
      // keys kb*32 + 8 g4 + 4h .. +3 of row n, from this wave's bias rows in the stage
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 bv = BT::read(Bs, n, kb * 32 + 8 * g4 + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sc[kb][4 * g4 + e] = __builtin_fmaf(sc[kb][4 * g4 + e], sl2, __builtin_fmaf(bv[e], kLog2e, nb0));
        }
    }
    if (masked) {
      // visible keys of this row inside the tile: tile-local [lo, hi). Register g of block
      // kb holds key kb*32 + res_row(g, h) = c + 4h with c a constant per register, so the
      // bounds are shifted by 4h once and each register compares its constant c.
      const int hi4 = min(min(ken, Nk), causal ? qrow + off + 1 : Nk) - kt0 - 4 * h;
      if (ranged) {
        const int lo4 = kst - kt0 - 4 * h;
        const unsigned span = (unsigned)max(hi4 - lo4, 0);  // c visible iff c - lo4 < span
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const int c = kb * 32 + res_row(g, 0);
            sc[kb][g] = (unsigned)(c - lo4) < span ? sc[kb][g] : kNegInf;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int g = 0; g < 16; ++g) {
            const int c = kb * 32 + res_row(g, 0);
            sc[kb][g] = c < hi4 ? sc[kb][g] : kNegInf;
          }
      }
    }
    u32x4 pb[KB][2];
    // probabilities 2^(x + sh) (packed into pb) and the lane's sum; sh moves the exponents
    // to a new running max (SH false: none)
    auto probs = [&](auto SH, float sh) __attribute__((always_inline)) -> float {
      float t = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int g = 8 * st + 2 * w;
            const float x0 = decltype(SH)::value ? sc[kb][g] + sh : sc[kb][g];
            const float x1 = decltype(SH)::value ? sc[kb][g + 1] + sh : sc[kb][g + 1];
            const float p0 = fast_exp2(x0), p1 = fast_exp2(x1);
            pb[kb][st][w] = E::pack2(p0, p1);
            t += p0 + p1;  // float32 row sum (the LSE needs the unrounded probabilities)
          }
      return t;
    };
    // move the running max to the row's max (both wave halves) and rescale; returns the
    // shift of the exponents to the new max
    auto remax = [&]() __attribute__((always_inline)) -> float {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int g = 0; g < 16; ++g) mx = __builtin_fmaxf(mx, sc[kb][g]);
      const float tmax = xhalf_max(mx) - nb0;  // the row's largest s * scale * log2(e) + bias
      const float mnew = __builtin_fmaxf(m2, tmax);
      const float alpha = mnew == kNegInf ? 1.f : fast_exp2(m2 - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m2 = mnew;
      return (mnew == kNegInf ? 0.f : -mnew) - nb0;
    };
    using NoShift = std::false_type;
    using Shift = std::true_type;
    float t;
    if (__builtin_expect(wave_any(m2 == kNegInf), 0)) {
      // a row without a finite running max yet: take the tile's max first
      t = probs(Shift{}, remax());
    } else {
      // Every row already holds a probability >= 1 (from the key that set m2), so the
      // tile needs no max of its own unless a score exceeds m2 + tau: then some p > 2^tau
      // and the lane's sum of p exceeds 2^tau too (an infinite p included). Only then is
      // the max taken, the accumulators rescaled and the tile's probabilities redone.
      t = probs(NoShift{}, 0.f);
      if (__builtin_expect(wave_any(!(t <= kTauP)), 0)) t = probs(Shift{}, remax());
    }
    l += t;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 vf[DB];  // V operands of this 16-key step, requested together
#pragma unroll
        for (int db = 0; db < DB; ++db) vf[db] = vfrag(Vs, db, kb, st);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = E::mma(vf[db], pb[kb][st], o[db]);
      }
  };

  // ---- main loop: ring of ST stages, P = ST-1 tiles in flight ------------------------
  // Ring position p (tile tile_at(p)) lives in stage p % ST.
  typename C::Tile dt;
  dt.init(wid, lane);
  auto issue = [&](auto J, int t) __attribute__((always_inline)) {
    char* sb = sptr(J);
    dt.load(K, t * BC, Nk, sb, wid);
    dt.load(V, t * BC, Nk, sb + C::Tile::kBytes, wid);
    if constexpr (TENSOR)
      BT::load(TB, a.tb_si, wq0, Nq, t * BC, Nk, sb + C::kStage + wid * BT::kWaveBytes, lane);
  };
  // wait until the oldest tile in flight has landed while `later` younger tiles may stay
  // in flight, then make every wave's part visible
  auto land = [&](int later) {
    if (P >= 3 && later >= 3) wait_vmem<(P >= 3 ? 3 : 0) * kOpsPerTile>();
    else if (P >= 2 && later == 2) wait_vmem<(P >= 2 ? 2 : 0) * kOpsPerTile>();
    else if (later == 1) wait_vmem<kOpsPerTile>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
  };
  // prologue: ring positions 0 .. P-1 (step p issues position p + P)
  if (0 < n_pos) issue(I0{}, tile_at(0));
  if constexpr (P >= 2) if (1 < n_pos) issue(I1{}, tile_at(1));
  if constexpr (P >= 3) if (2 < n_pos) issue(I2{}, tile_at(2));
  // The Q fragments and every prologue tile land. Waiting for all of them (rather than
  // for the first tile only) leaves no register load outstanding in the loop, so the
  // compiler puts no full vector-memory wait, which would also wait for the ring's loads
  // in flight, in front of the loop's MFMAs.
  wait_vmem<0>();
  __builtin_amdgcn_s_barrier();
  int n_comp = 0;  // tiles this wave computes (wave-uniform; reported with a.counts)
  auto step = [&](auto J, int p) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    if constexpr (SPARSE) lw.slide(p);
    const int t = tile_at(p);
    // the stage of position p+P held position p-1, which every wave finished before the
    // barrier
    if (p + P < n_pos) issue(std::integral_constant<int, j + P>{}, tile_at(p + P));
    sync_check();
    if (wave_needs(p, t)) {
      ++n_comp;
      const char* sb = sptr(J);
      tile(sb, sb + C::Tile::kBytes, sb + C::kStage + wid * BT::kWaveBytes, t * BC, !full_tile(t));
    }
    if (p + 1 < n_pos) land(min(p + P, n_pos - 1) - (p + 1));
  };
  for (int p = 0; p < n_pos; p += ST) {
    step(I0{}, p);
    if (p + 1 < n_pos) step(I1{}, p + 1);
    if constexpr (ST > 2) if (p + 2 < n_pos) step(I2{}, p + 2);
    if constexpr (ST > 3) if (p + 3 < n_pos) step(I3{}, p + 3);
  }

  // ---- epilogue -----------------------------------------------------------------------
  if (a.counts != nullptr && lane == 0) {
    atomicAdd(&a.counts[1], (unsigned long long)n_comp);
    if (wid == 0) atomicAdd(&a.counts[0], (unsigned long long)n_pos);
  }
  const float lt = xhalf_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (a.n_split > 1) {
    // normalised float32 partial of this key range and its LSE (nothing visible in the
    // range: O = 0, LSE = -inf, which gives it zero weight in the merge)
    if (qrow < Nq) {
      const size_t rows = (size_t)a.B * a.H * Nq;
      const size_t row = (size_t)split * rows + (size_t)bh * Nq + qrow;
      float* op = a.o_part + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * h;
          *reinterpret_cast<f32x4*>(op + d0) =
              f32x4{o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv,
                    o[db][4 * g4 + 3] * inv};
        }
      if (h == 0)
        a.lse_part[row] = lt > 0.f ? (m2 + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
    }
  } else if (qrow < Nq) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * h;
        stg8(O + (size_t)qrow * D + d0,
             u32x2{E::pack2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                   E::pack2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)});
      }
    if (h == 0 && a.lse != nullptr)
      a.lse[(size_t)bh * Nq + qrow] = lt > 0.f ? (m2 + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------------
// key-range summary: out[4r..4r+3] = min/max of clamped start and end over rows of block r
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mask_summary_kernel(const int32_t* __restrict__ ks,
                                                           const int32_t* __restrict__ ke,
                                                           int Nq, int Nk, int block,
                                                           int32_t* __restrict__ out) {
  __shared__ int red[4][4];
  const int r = blockIdx.x;
  const int r0 = r * block, r1 = min(Nq, r0 + block);
  int mn_s = Nk, mx_s = 0, mn_e = Nk, mx_e = 0;
  for (int i = r0 + (int)threadIdx.x; i < r1; i += 256) {
    const int s = min(max(ks[i], 0), Nk), e = min(max(ke[i], 0), Nk);
    mn_s = min(mn_s, s); mx_s = max(mx_s, s); mn_e = min(mn_e, e); mx_e = max(mx_e, e);
  }
  mn_s = wave_min(mn_s); mx_s = wave_max(mx_s); mn_e = wave_min(mn_e); mx_e = wave_max(mx_e);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[w][0] = mn_s; red[w][1] = mx_s; red[w][2] = mn_e; red[w][3] = mx_e; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 4; ++i) {
      red[0][0] = min(red[0][0], red[i][0]); red[0][1] = max(red[0][1], red[i][1]);
      red[0][2] = min(red[0][2], red[i][2]); red[0][3] = max(red[0][3], red[i][3]);
    }
    for (int i = 0; i < 4; ++i) out[4 * r + i] = red[0][i];
  }
}

hipError_t launch_mask_summary(const int32_t* ks, const int32_t* ke, int Nq, int Nk, int block,
                               int32_t* out, hipStream_t st) {
  const int nb = (Nq + block - 1) / block;
  hipLaunchKernelGGL(mask_summary_kernel, dim3(nb), dim3(256), 0, st, ks, ke, Nq, Nk, block, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// tile configurations per (dtype, d) and the launcher
// ---------------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_merge(const FwdArgs& a, hipStream_t st);

template <typename T, int D, int BC, int QSUB, int NW, int WPE>
static hipError_t launch_cfg(int bias, FwdArgs& a, hipStream_t st) {
  using C = FwdCfg<T, D, BC, QSUB, NW>;
  static_assert(kFwdTileKeys % BC == 0, "split ranges are whole tiles");
  a.nqb = (a.Nq + C::kBR - 1) / C::kBR;
  if (a.n_split < 1) a.n_split = 1;
  const int BH = a.B * a.H;
  a.sched = (BH % 8 == 0) ? kSchedXcdLpt : kSchedHeadMajor;
  const dim3 grid((unsigned)(BH * a.nqb * a.n_split)), block(C::kNT);
  if (bias == kBiasTensor)
    hipLaunchKernelGGL((fwd_kernel<T, D, BC, QSUB, NW, WPE, kBiasTensor>), grid, block, 0, st, a);
  else if (bias)
    hipLaunchKernelGGL((fwd_kernel<T, D, BC, QSUB, NW, WPE, kBiasSlope>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, BC, QSUB, NW, WPE, kBiasNone>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  return launch_merge<T, D>(a, st);
}

// ---------------------------------------------------------------------------------
// Merge of split-key partials: LSE = log sum_r exp(LSE_r), O = sum_r exp(LSE_r - LSE) O_r.
// D/4 threads per row, one float4 of the row each; n_split <= ceil(N_k / 64).
// ---------------------------------------------------------------------------------
// four merged output values in the output type (16-bit: rounded to nearest even)
template <typename T>
__device__ inline void store_merged(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    using E = Elt<T>;
    stg8(p, u32x2{E::pack2(v[0], v[1]), E::pack2(v[2], v[3])});
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        T* __restrict__ o, float* __restrict__ lse,
                                                        int rows, int n_split) {
  constexpr int TPR = D / 4, RPB = 256 / TPR;
  const int r = blockIdx.x * RPB + (int)threadIdx.x / TPR;
  const int c = ((int)threadIdx.x % TPR) * 4;
  if (r >= rows) return;
  float m = kNegInf;
  for (int s = 0; s < n_split; ++s) m = __builtin_fmaxf(m, lse_part[(size_t)s * rows + r]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < n_split; ++s) {
      const float ls = lse_part[(size_t)s * rows + r];
      if (ls == kNegInf) continue;  // nothing visible in that range
      const float w = fast_exp2((ls - m) * kLog2e);
      den += w;
      const f32x4 x = *reinterpret_cast<const f32x4*>(o_part + ((size_t)s * rows + r) * D + c);
      acc += w * x;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  store_merged(o + (size_t)r * D + c, acc * inv);
  if (c == 0 && lse != nullptr)
    lse[r] = den > 0.f ? m + __builtin_amdgcn_logf(den) * kLn2 : kNegInf;
}

// The same merge with one workgroup per row, for many ranges: D/4 threads per group, G
// groups; group g takes ranges g, g + G, ... (their loads are independent, so they
// overlap), and the G partial sums are added in group order through LDS. With one
// thread per float4 of a row and 64 ranges, the loop above waits for 64 loads one
// after the other, which is most of a decode step with few heads.
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_merge_wide_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ lse_part,
                                                             T* __restrict__ o,
                                                             float* __restrict__ lse, int rows,
                                                             int n_split) {
  constexpr int TPR = D / 4, G = 256 / TPR;
  __shared__ float wmax[4];
  __shared__ f32x4 acc_s[G][TPR];
  __shared__ float den_s[G];
  const int r = blockIdx.x, tid = threadIdx.x, g = tid / TPR, t = tid % TPR, c = 4 * t;
  float m = kNegInf;
  for (int s = tid; s < n_split; s += 256) m = __builtin_fmaxf(m, lse_part[(size_t)s * rows + r]);
  m = wave_fmax(m);
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != kNegInf) {
    for (int s = g; s < n_split; s += G) {
      const float ls = lse_part[(size_t)s * rows + r];
      if (ls == kNegInf) continue;  // nothing visible in that range
      const float w = fast_exp2((ls - m) * kLog2e);
      den += w;
      const f32x4 x = *reinterpret_cast<const f32x4*>(o_part + ((size_t)s * rows + r) * D + c);
      acc += w * x;
    }
  }
  acc_s[g][t] = acc;
  if (t == 0) den_s[g] = den;
  __syncthreads();
  if (g != 0) return;
  for (int j = 1; j < G; ++j) {
    acc += acc_s[j][t];
    den += den_s[j];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  store_merged(o + (size_t)r * D + c, acc * inv);
  if (t == 0 && lse != nullptr)
    lse[r] = den > 0.f ? m + __builtin_amdgcn_logf(den) * kLn2 : kNegInf;
}

// Up to kMergeRowsSplit ranges: one thread per float4 of a row; more: a workgroup per row.
constexpr int kMergeRowsSplit = 4;

template <typename T, int D>
static hipError_t launch_merge(const FwdArgs& a, hipStream_t st) {
  const int rows = a.B * a.H * a.Nq;
  if (a.n_split > kMergeRowsSplit) {
    hipLaunchKernelGGL((fwd_merge_wide_kernel<T, D>), dim3((unsigned)rows), dim3(256), 0, st,
                       a.o_part, a.lse_part, static_cast<T*>(a.o), a.lse, rows, a.n_split);
    return hipGetLastError();
  }
  constexpr int RPB = 256 / (D / 4);
  hipLaunchKernelGGL((fwd_merge_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                     0, st, a.o_part, a.lse_part, static_cast<T*>(a.o), a.lse, rows, a.n_split);
  return hipGetLastError();
}

// float32 configurations (d, BC keys per tile, QSUB 32-row sub-blocks per wave, NW waves,
// waves per SIMD); 16-bit types use fwd16_kernel below
#define FA_FWD_CFG_32_D128 128, 32, 1, 4, 1
#define FA_FWD_CFG_32_D64 64, 32, 1, 4, 1


template <typename T, int D, int BC, int NW, int ST>
static hipError_t launch16(int bias, FwdArgs& a, hipStream_t st) {
  using C = Fwd16Cfg<D, BC, NW, ST>;
  static_assert(kFwdTileKeys % BC == 0, "split ranges are whole tiles");
  a.nqb = (a.Nq + C::kBR - 1) / C::kBR;
  a.rows_wg = C::kBR;
  a.keys_tile = BC;
  if (a.n_split < 1) a.n_split = 1;
  const int BH = a.B * a.H;
  a.sched = (BH % 8 == 0) ? kSchedXcdLpt : kSchedHeadMajor;
  const dim3 grid((unsigned)(BH * a.nqb * a.n_split)), block(C::kNT);
  const bool sparse = a.bmask != nullptr;
  if (bias == kBiasTensor) {
    // (the bias tensor's tile rides in a two-stage ring)
    if constexpr (ST == 2 && NW == 4) {
      if (sparse)
        hipLaunchKernelGGL((fwd16_kernel<T, D, BC, NW, ST, kBiasTensor, true>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((fwd16_kernel<T, D, BC, NW, ST, kBiasTensor, false>), grid, block, 0, st, a);
    } else {
      return hipErrorNotSupported;
    }
  } else if (bias && sparse)
    hipLaunchKernelGGL((fwd16_kernel<T, D, BC, NW, ST, kBiasSlope, true>), grid, block, 0, st, a);
  else if (bias)
    hipLaunchKernelGGL((fwd16_kernel<T, D, BC, NW, ST, kBiasSlope, false>), grid, block, 0, st, a);
  else if (sparse)
    hipLaunchKernelGGL((fwd16_kernel<T, D, BC, NW, ST, kBiasNone, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((fwd16_kernel<T, D, BC, NW, ST, kBiasNone, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  return launch_merge<T, D>(a, st);
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// 16-bit configurations.
//   d = 64: 4 waves x 32 rows, 64-key tiles, 4 stages (64 KB).
//   d = 128, few query rows split over key ranges: 4 waves, 32-key tiles, 4 stages
//     (64 KB: two workgroups, i.e. two computing waves, per compute unit).
//   d = 128 otherwise: 8 waves x 32 rows, 64-key tiles; 4 stages (128 KB) when a head has
//     at most kFwdFewRows rows (decode-like: the load of every key is compulsory and a
//     deeper ring hides more of it), else 2 stages (64 KB: one tile in flight measured
//     3-4 % faster than three on the causal N = 8192 shape). When a head has more than
//     kFwdFewRows rows and the grid has fewer than four such 256-row units per compute
//     unit, or rows carry key ranges (whose visible tiles smaller blocks follow more
//     closely): 4 waves x 32 rows with 2 stages (64 KB, two workgroups per compute unit),
//     where twice as many, fuller blocks balance the load better.
// For N_q <= kFwdFewRows every d = 128 variant holds the whole head in one query block.
// With a bias tensor, whose tile (4 waves x 32 rows x the tile's keys, float32) shares
// each stage with K and V: 4 waves, two stages, 32-key tiles (d = 128: 67 KB, two
// workgroups per compute unit; d = 64: 51 KB). The bias makes the kernel wait on HBM;
// a second workgroup per compute unit hides it better than 64-key tiles at one
// workgroup (134 KB): 503-510 against 649-667 us on the bf16 B2 H8 N8192 d128
// key-range workload with a [1, H, N, N] bias.
template <typename T>
static hipError_t launch16_for(int d, int bias, FwdArgs& a, hipStream_t st) {
  if (bias == kBiasTensor) {
    if (d == 64) return launch16<T, 64, 32, 4, 2>(bias, a, st);
    return launch16<T, 128, 32, 4, 2>(bias, a, st);
  }
  if (d == 64) return launch16<T, 64, 64, 4, 4>(bias, a, st);
  if (a.Nq <= kFwdFewRows) {
    if (a.n_split > 1) return launch16<T, 128, 32, 4, 4>(bias, a, st);
    return launch16<T, 128, 64, 8, 4>(bias, a, st);
  }
  const long long units256 =
      (long long)a.B * a.H * ((a.Nq + 255) / 256) * (a.n_split > 1 ? a.n_split : 1);
  if (a.key_start != nullptr || units256 < 4LL * device_cus())
    return launch16<T, 128, 64, 4, 2>(bias, a, st);
  return launch16<T, 128, 64, 8, 2>(bias, a, st);
}

hipError_t launch_fwd(fa_dtype dt, int d, int bias, FwdArgs& a, hipStream_t st) {
  switch (dt) {
    case FA_BF16:
      return launch16_for<__bf16>(d, bias, a, st);
    case FA_F16:
      return launch16_for<_Float16>(d, bias, a, st);
    case FA_F32:
      return d == 128 ? launch_cfg<float, FA_FWD_CFG_32_D128>(bias, a, st)
                      : launch_cfg<float, FA_FWD_CFG_32_D64>(bias, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
