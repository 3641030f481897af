// fa_fp8.hip -- FP8 (OCP E4M3) forward with block quantisation and incoherent processing.
//
// Source: marketmaker.cc blog on Flash Attention ("Apakah Konteks Sehari Penuh ..."),
// section "FA3: Mekanika hopper", item 3: FP8 doubles the matrix rate; outliers spoil
// plain FP8 attention; a random rotation of the vectors before block quantisation
// spreads an outlier's magnitude over all coordinates.
//
// Quantiser: one workgroup per 64-row block of one (b, h). Q and K may be rotated by
// diag(signs) H_d (H_d the Sylvester Hadamard matrix; the 1/sqrt(d) factor is left to
// the scores): the fast Walsh-Hadamard transform runs in float64, where the sums of d
// 16-bit inputs are exact, and is rounded once to float32. Each 64-row block gets
// amax = max |x|; Q and K codes are RNE(clamp(x * (448 / amax))), V codes RNE(x * 2^-e)
// with 2^e the smallest power of two such that amax <= 448 * 2^e, the block scale the
// P V product applies itself. Q is stored row-major; K and V are stored as the LDS images
// of the forward's tiles (see fa.h), so the forward copies them with plain linear direct
// loads.
//
// Forward: the 16-bit forward's structure (query rows per wave, online softmax with
// lazy rescale, K/V tiles through a ring of LDS stages by direct loads) with
// v_mfma_f32_32x32x64_f8f6f4 for S^T = K Q^T (k = 64 bytes of d per step) and for
// O^T += V^T P^T (k = all 64 keys of a tile in one step, with the tile's V block scale
// given to the product as its E8M0 operand scale). The probabilities (at most 2^8 with
// the lazy rescale) are rounded to E4M3 straight from the score registers; the
// transposed, key-permuted V tile puts each lane's 32 keys in the same byte order.
#include <hip/hip_runtime.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4m3Max = 448.f;

// Exponent e of a V block's scale 2^e: the smallest e >= -127 (the E8M0 floor) with
// amax <= 448 * 2^e, and 0 for an all-zero block. With 448 = 1.75 * 2^8 and amax =
// 1.m * 2^(E - 127) (E its biased exponent field) that is E - 135, plus one when the
// mantissa exceeds 1.75 (field above 0x600000).
__device__ inline int v_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int eb = (int)(b >> 23);
  if (eb == 0) return -127;  // subnormal: below 2^-126 < 448 * 2^-127
  return max(eb - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0), -127);
}

// ---------------------------------------------------------------------------------
// byte layouts of the quantised K and V tiles (64 rows of one (b, h))
// ---------------------------------------------------------------------------------
// K tile: row r (key) at r * D bytes, 16-byte chunk c of the row in slot c ^ k_swz(r):
// the 16 lanes of a row read (rows r..r+15, one chunk) then hit 16 distinct bank groups.
template <int D>
__device__ __host__ constexpr int k_swz(int r) { return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3; }
// V tile: transposed, row e (d column) of 64 bytes; byte position p holds key kappa(p),
// the order in which a lane of the P^T operand holds its keys; chunk c of the row in
// slot c ^ ((e >> 2) & 3).
__device__ __host__ constexpr int v_pos(int key) {  // inverse of kappa
  const int kh = key >> 5, j = key & 31;
  return 32 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3) + 16 * kh;
}
__device__ __host__ constexpr int v_byte(int e, int key) {
  const int p = v_pos(key);
  return e * 64 + 16 * ((p >> 4) ^ ((e >> 2) & 3)) + (p & 15);
}

// ---------------------------------------------------------------------------------
// quantiser
// ---------------------------------------------------------------------------------
template <typename T, int D>
__device__ inline void load_quarter_row(const T* row, int q, double (&v)[D / 4]) {
  constexpr int PER = D / 4;
#pragma unroll
  for (int c = 0; c < PER / 8; ++c) {
    const u32x4 w = ldg16(row + q * PER + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = w[i];
      v[8 * c + 2 * i] = (double)Elt<T>::to_f32(x & 0xffffu);
      v[8 * c + 2 * i + 1] = (double)Elt<T>::to_f32(x >> 16);
    }
  }
}

// Rotation of one row held by a quad of lanes (lane quarter q holds elements
// q*PER .. q*PER+PER-1): element-wise signs, then the Walsh-Hadamard butterflies
// (a, b) -> (a + b, a - b) over strides 1, 2, ..., D/2; the last two strides pair lanes.
template <int D>
__device__ inline void fwht_row(double (&v)[D / 4], int q, const uint32_t* sign_bits) {
  constexpr int PER = D / 4;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = q * PER + i;
    if ((sign_bits[e >> 5] >> (e & 31)) & 1u) v[i] = -v[i];
  }
#pragma unroll
  for (int s = 1; s < PER; s <<= 1)
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (!(i & s)) {
        const double x = v[i], y = v[i + s];
        v[i] = x + y;
        v[i + s] = x - y;
      }
#pragma unroll
  for (int s = 1; s < 4; s <<= 1)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const double p = __shfl_xor(v[i], s);
      v[i] = (q & s) ? p - v[i] : v[i] + p;
    }
}

__device__ inline float block_max256(float x, float* red) {
  x = wave_fmax(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  return r;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const Fp8QuantArgs a) {
  constexpr int PER = D / 4;
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t vt[64 * D];  // V tile image
  const int nb = a.Np / 64;
  const int bh = blockIdx.x / nb, blk = blockIdx.x - bh * nb;
  const int r = threadIdx.x >> 2, q = threadIdx.x & 3, row = blk * 64 + r;
  double v[PER];
  if (row < a.N) {
    load_quarter_row<T, D>(static_cast<const T*>(a.x) + ((size_t)bh * a.N + row) * D, q, v);
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = 0.0;
  }
  if (a.rotate) fwht_row<D>(v, q, a.sign_bits);
  float f[PER];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    f[i] = (float)v[i];  // one rounding of the exact value
    m = __builtin_fmaxf(m, __builtin_fabsf(f[i]));
  }
  const float amax = block_max256(m, red);
  if (threadIdx.x == 0) a.amax[(size_t)bh * nb + blk] = amax;
  // Q, K: x * (448 / amax); V: x * 2^-e, exact (127 - e lies in [7, 254], a normal float)
  const float inv = a.layout == FA_FP8_V
                        ? __uint_as_float((uint32_t)(127 - v_block_exp(amax)) << 23)
                        : (amax > 0.f ? kE4m3Max / amax : 0.f);
  uint32_t w[PER / 4];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = __builtin_fminf(__builtin_fmaxf(f[4 * i + j] * inv, -kE4m3Max), kE4m3Max);
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
    w[i] = (uint32_t)pk;
  }
  uint8_t* out = a.x8 + ((size_t)bh * a.Np + (size_t)blk * 64) * D;  // this block's 64 rows
  if (a.layout == FA_FP8_Q) {
    uint8_t* p = out + r * D + q * PER;
#pragma unroll
    for (int c = 0; c < PER / 16; ++c)
      *reinterpret_cast<u32x4*>(p + 16 * c) = u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
  } else if (a.layout == FA_FP8_K) {
#pragma unroll
    for (int c = 0; c < PER / 16; ++c) {
      const int chunk = q * (PER / 16) + c;
      *reinterpret_cast<u32x4*>(out + r * D + 16 * (chunk ^ k_swz<D>(r))) =
          u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
    }
  } else {
    // V: scatter the bytes into the tile image in LDS, then copy it out linearly
#pragma unroll
    for (int i = 0; i < PER; ++i)
      vt[v_byte(q * PER + i, r)] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 64 * D / 4096; ++c) {
      const int off = 4096 * c + 16 * threadIdx.x;
      *reinterpret_cast<u32x4*>(out + off) = *reinterpret_cast<const u32x4*>(vt + off);
    }
  }
}

// ---------------------------------------------------------------------------------
// FP8 forward
// ---------------------------------------------------------------------------------
__device__ inline f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  // A and B in E4M3 (format code 0), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// the same with E8M0 operand scales: A times 2^(sa - 127), B times 2^(sb - 127) (byte 0 of
// each; every lane passes the same value here). Both must be run-time values: a constant
// scale operand would be encoded as a float32 constant.
__device__ inline f32x16 mma8s(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ inline i32x8 cat8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <typename T, int D, int NW, int ST>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(2, 2)))
void fwd8_kernel(const Fp8FwdArgs a) {
  using E = Elt<T>;
  constexpr int TB = 64 * D;              // bytes of a K (or V) tile
  constexpr int kStage = 2 * TB;          // K tile, then V tile
  constexpr int DC = D / 64;              // 64-byte k-steps of S^T over d
  constexpr int DB = D / 32;              // 32-wide d blocks of O^T
  constexpr int kOpsPerWave = 2 * TB / 1024 / NW;  // 1 KB direct loads per wave per tile
  constexpr int P = ST - 1;
  static_assert(kOpsPerWave >= 1 && kOpsPerWave * NW * 1024 == 2 * TB, "tile split over waves");
  static_assert(ST >= 2 && ST <= 4 && ST * kStage <= 160 * 1024, "LDS ring");
  __shared__ __attribute__((aligned(1024))) char stg0[kStage];
  __shared__ __attribute__((aligned(1024))) char stg1[kStage];
  __shared__ __attribute__((aligned(1024))) char stg2[ST > 2 ? kStage : 1];
  __shared__ __attribute__((aligned(1024))) char stg3[ST > 3 ? kStage : 1];
  __shared__ int wg_hi[NW];
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

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int n = lane & 31, h = lane >> 5;
  const int Nq = a.Nq, Nk = a.Nk, off = Nk - Nq;
  const bool causal = a.causal != 0;
  int bh, qb;
  map_block(blockIdx.x, a.B * a.H, a.nqb, a.sched, true, bh, qb);
  const uint8_t* Q8 = a.q8 + (size_t)bh * a.Nqp * D;
  const uint8_t* K8 = a.k8 + (size_t)bh * a.Nkp * D;
  const uint8_t* V8 = a.v8 + (size_t)bh * a.Nkp * D;
  // K block amaxes through the constant address space: a wave-uniform index then gives
  // a scalar load, whose wait does not cover the ring's direct loads in flight
  const __attribute__((address_space(4))) float* kam =
      (const __attribute__((address_space(4))) float*)(a.k_amax + (size_t)bh * (a.Nkp / 64));
  T* O = static_cast<T*>(a.o) + (size_t)bh * Nq * D;

  const int wq0 = qb * 32 * NW + 32 * wid, qrow = wq0 + n;
  const bool wave_live = wq0 < Nq;
  const int wq_last = min(wq0 + 32, Nq) - 1;
  int w_hi = Nk, w_full_c = Nk;
  if (causal) {
    w_hi = min(Nk, wq_last + off + 1);
    w_full_c = max(0, min(Nk, wq0 + off + 1));
  }
  if (!wave_live || w_hi <= 0) w_hi = 0;
  // V block amaxes the same way: tile t's block scale exponent for the P V product
  const __attribute__((address_space(4))) float* vam =
      (const __attribute__((address_space(4))) float*)(a.v_amax + (size_t)bh * (a.Nkp / 64));
  int e8_one = 127;  // E8M0 for 2^0, kept opaque to the compiler (see mma8s)
  asm volatile("" : "+v"(e8_one));
  if (lane == 0) wg_hi[wid] = w_hi;
  __syncthreads();
  int g_hi = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) g_hi = max(g_hi, wg_hi[w]);
  const int n_t = (g_hi + 63) / 64;
  auto live_tile = [&](int t) { return t * 64 < w_hi; };
  auto full_tile = [&](int t) { return (t + 1) * 64 <= Nk && (t + 1) * 64 <= w_full_c; };

  // the score scale of this wave's rows: scale * log2(e) (/ d if rotated) * q block scale
  const float sq = wave_live ? a.q_amax[(size_t)bh * (a.Nqp / 64) + wq0 / 64] / kE4m3Max : 0.f;
  const float csq = a.sl2 * sq;

  // Q operand (B of S^T = K Q^T): query row n, bytes 64c + 32h .. +31 of each k-step
  i32x8 qf[DC];
  if (wave_live) {
    const uint8_t* qp = Q8 + (size_t)qrow * D + 32 * h;
#pragma unroll
    for (int c = 0; c < DC; ++c) qf[c] = cat8(ldg16(qp + 64 * c), ldg16(qp + 64 * c + 16));
  } else {
#pragma unroll
    for (int c = 0; c < DC; ++c) qf[c] = i32x8{};
  }

  // per-lane LDS offsets: K row 32kh + n, chunks 4c + 2h, +1 (swizzled); V^T row
  // 32db + n, chunks 2h, 2h + 1 (swizzled)
  int ka[DC][2];
#pragma unroll
  for (int c = 0; c < DC; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) ka[c][j] = n * D + 16 * (((D / 16 / DC) * c + 2 * h + j) ^ k_swz<D>(n));
  int va[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) va[j] = TB + n * 64 + 16 * ((2 * h + j) ^ ((n >> 2) & 3));

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m2 = kNegInf, l = 0.f;

  auto tile = [&](const char* sb, int t, bool masked) __attribute__((always_inline)) {
    const int kt0 = t * 64;
    f32x16 sc[2];
    {
      i32x8 kf[2][DC];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int c = 0; c < DC; ++c)
          kf[kh][c] = cat8(lds_ld16(sb, kh * 32 * D + ka[c][0]), lds_ld16(sb, kh * 32 * D + ka[c][1]));
      sched_fence();
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        sc[kh] = f32x16{};
#pragma unroll
        for (int c = 0; c < DC; ++c) sc[kh] = mma8(kf[kh][c], qf[c], sc[kh]);
      }
    }
    // this tile's score scale; kept positive so that a masked -inf never meets a zero
    const float ct = __builtin_fmaxf(csq * (kam[t] / kE4m3Max), 1.17549435e-38f);
    if (masked) {
      const int hi = min(Nk, causal ? qrow + off + 1 : Nk) - kt0;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int g = 0; g < 16; ++g)
          sc[kh][g] = (kh * 32 + res_row(g, h) < hi) ? sc[kh][g] : kNegInf;
    }
    // probabilities (<= 2^8) rounded to E4M3, packed in key order kappa: bytes 0-15 from
    // the first 32-key block, 16-31 from the second; returns the lane's sum
    i32x8 pf;
    auto probs = [&]() __attribute__((always_inline)) -> float {
      const float nb = m2 == kNegInf ? 0.f : -m2;
      float t = 0.f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int g = 4 * w;
          const float p0 = fast_exp2(__builtin_fmaf(sc[kh][g], ct, nb));
          const float p1 = fast_exp2(__builtin_fmaf(sc[kh][g + 1], ct, nb));
          const float p2 = fast_exp2(__builtin_fmaf(sc[kh][g + 2], ct, nb));
          const float p3 = fast_exp2(__builtin_fmaf(sc[kh][g + 3], ct, nb));
          t += (p0 + p1) + (p2 + p3);
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, pk, true);
          pf[4 * kh + w] = pk;
        }
      return t;
    };
    // moves the running max to the row's max (both wave halves) and rescales
    auto remax = [&]() __attribute__((always_inline)) {
      float mx = kNegInf;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int g = 0; g < 16; ++g) mx = __builtin_fmaxf(mx, sc[kh][g]);
      const float tmax = xhalf_max(mx * ct);
      const float mnew = __builtin_fmaxf(m2, tmax);
      const float alpha = mnew == kNegInf ? 1.f : fast_exp2(m2 - mnew);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m2 = mnew;
    };
    // A row with a finite running max holds a probability >= 1 already, so the tile's max
    // is only needed when a score exceeds m2 + tau: then some p > 2^tau and the lane's sum
    // exceeds 2^tau too. Rows without a finite max yet take the max first.
    float tsum;
    if (__builtin_expect(wave_any(m2 == kNegInf), 0)) {
      remax();
      tsum = probs();
    } else {
      tsum = probs();
      if (__builtin_expect(wave_any(!(tsum <= kTauP)), 0)) {
        remax();
        tsum = probs();
      }
    }
    l += tsum;
    i32x8 vf[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vf[db] = cat8(lds_ld16(sb, db * 32 * 64 + va[0]), lds_ld16(sb, db * 32 * 64 + va[1]));
    const int e8_v = v_block_exp(vam[t]) + 127;  // V block scale 2^e as E8M0
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = mma8s(vf[db], pf, o[db], e8_v, e8_one);
  };

  // ring: tile t's K and V images copied linearly, stage t % ST
  auto issue = [&](auto J, int t) __attribute__((always_inline)) {
    char* sb = sptr(J);
#pragma unroll
    for (int j = 0; j < kOpsPerWave; ++j) {
      const int u = wid * kOpsPerWave + j;  // 1 KB window of the stage (wave-uniform)
      const uint8_t* g = u * 1024 < TB ? K8 + (size_t)t * TB + u * 1024
                                       : V8 + (size_t)t * TB + (u * 1024 - TB);
      DmaBase<true>(g).load<16>(16u * (uint32_t)lane, sb + u * 1024);
    }
  };
  auto land = [&](int later) {
    if (P >= 3 && later >= 3) wait_vmem<(P >= 3 ? 3 : 0) * kOpsPerWave>();
    else if (P >= 2 && later == 2) wait_vmem<(P >= 2 ? 2 : 0) * kOpsPerWave>();
    else if (later == 1) wait_vmem<kOpsPerWave>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
  };
  // prologue: tiles 0 .. P-1 (step t issues tile t + P)
  if (0 < n_t) issue(I0{}, 0);
  if constexpr (P >= 2) if (1 < n_t) issue(I1{}, 1);
  if constexpr (P >= 3) if (2 < n_t) issue(I2{}, 2);
  wait_vmem<0>();
  __builtin_amdgcn_s_barrier();
  auto step = [&](auto J, int t) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    if (t + P < n_t) issue(std::integral_constant<int, j + P>{}, t + P);
    sync_check();
    if (live_tile(t)) tile(sptr(J), t, !full_tile(t));
    if (t + 1 < n_t) land(min(t + P, n_t - 1) - (t + 1));
  };
  for (int t = 0; t < n_t; t += ST) {
    step(I0{}, t);
    if (t + 1 < n_t) step(I1{}, t + 1);
    if constexpr (ST > 2) if (t + 2 < n_t) step(I2{}, t + 2);
    if constexpr (ST > 3) if (t + 3 < n_t) step(I3{}, t + 3);
  }

  // epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
  const float lt = xhalf_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow < Nq) {
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
// launchers
// ---------------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_quant_t(Fp8QuantArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H * (a.Np / 64))), block(256);
  hipLaunchKernelGGL((fp8_quant_kernel<T, D>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fp8_quant(fa_dtype dt, int d, Fp8QuantArgs& a, hipStream_t st) {
  if (dt == FA_BF16) return d == 128 ? launch_quant_t<__bf16, 128>(a, st) : launch_quant_t<__bf16, 64>(a, st);
  return d == 128 ? launch_quant_t<_Float16, 128>(a, st) : launch_quant_t<_Float16, 64>(a, st);
}

template <typename T, int D>
static hipError_t launch_fwd8_t(Fp8FwdArgs& a, hipStream_t st) {
  // 4 waves x 32 rows, one tile in flight (measured on the bf16 causal N = 8192 d = 128
  // shape: 344 us, against 353 us with 2 or 3 tiles in flight and 370-386 us with 8 waves)
  constexpr int NW = 4, ST = 2;
  a.nqb = (a.Nq + 32 * NW - 1) / (32 * NW);
  a.sched = ((a.B * a.H) % 8 == 0) ? kSchedXcdLpt : kSchedHeadMajor;
  const dim3 grid((unsigned)(a.B * a.H * a.nqb)), block(NW * 64);
  hipLaunchKernelGGL((fwd8_kernel<T, D, NW, ST>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd8(fa_dtype out, int d, Fp8FwdArgs& a, hipStream_t st) {
  if (out == FA_BF16) return d == 128 ? launch_fwd8_t<__bf16, 128>(a, st) : launch_fwd8_t<__bf16, 64>(a, st);
  return d == 128 ? launch_fwd8_t<_Float16, 128>(a, st) : launch_fwd8_t<_Float16, 64>(a, st);
}

}  // namespace fa
