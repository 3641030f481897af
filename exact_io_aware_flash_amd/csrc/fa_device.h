// fa_device.h -- device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA conventions used throughout (32x32 tiles, one wave = 64 lanes, lane = 32*h + n):
//   A operand (M x K):  lane n + 32*h holds row n and the K-slice owned by half h;
//   B operand (K x N):  lane n + 32*h holds column n and the same K-slice of half h;
//   result (M x N):     lane n + 32*h, register g holds row 8*(g/4) + 4*h + (g%4), column n.
// For bf16/f16 (v_mfma_f32_32x32x16_*) the K-slice is 8 elements (half h: k = 8h..8h+7);
// for f32 (v_mfma_f32_32x32x2_f32) it is one element (k = h). A and B always share the
// K-slice mapping, so any consistent relabelling of K on both operands gives the same
// product; the kernels use this to feed probabilities straight from the result registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// Lazy rescale of the online softmax: the running max (log2 units) only moves when a
// row's new scores exceed it by more than kTau, so probabilities stay <= 2^kTau.
constexpr float kTau = 8.0f;
constexpr float kTauP = 256.0f;  // 2^kTau: a probability above it means the max moved

// Element-type traits: 16-bit types go through the 32x32x16 MFMA, float through 32x32x2.
template <typename T> struct Elt;

template <> struct Elt<__bf16> {
  static constexpr int kBytes = 2;
  // acc + lo(w) + hi(w) for a word of two packed elements (v_dot2c_f32_bf16 with 1.0)
  __device__ static inline float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
  }
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 (round to nearest even) packed low|high
  __device__ static inline uint32_t pack2(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  // the element in the low 16 bits of `bits`, widened exactly
  __device__ static inline float to_f32(uint32_t bits) { return __builtin_bit_cast(float, bits << 16); }
};

template <> struct Elt<_Float16> {
  static constexpr int kBytes = 2;
  __device__ static inline float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                  __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
  }
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
  }
};

template <> struct Elt<float> {
  static constexpr int kBytes = 4;
  __device__ static inline f32x16 mma1(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Result-register helpers for the 32x32 layout.
__device__ constexpr int res_row(int g, int h) { return 8 * (g / 4) + 4 * h + (g % 4); }

// Cross-half exchange: value held by lane l ^ 32 (the other half of the same column),
// one ds_bpermute with the byte address 4 * (l ^ 32).
__device__ inline int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
__device__ inline float xhalf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2,
                                                                __builtin_bit_cast(int, v)));
}

__device__ inline float xhalf_max(float v) { return __builtin_fmaxf(v, xhalf(v)); }
__device__ inline float xhalf_sum(float v) { return v + xhalf(v); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exponent offset of a row in the recomputed probabilities of the backward passes,
// p = exp2(s * scale * log2(e) + bias * log2(e) - offset). A row with no visible key has
// LSE = -inf (its output is 0); its offset is +inf, so every probability of the row is
// exactly 0 whatever the bias (-inf - (-inf) would be NaN, and a finite score minus -inf
// would be +inf).
__device__ inline float lse_offset2(float lse) { return lse == kNegInf ? -kNegInf : lse * kLog2e; }

__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// 16-byte global load/store through plain vector accesses.
__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void stg8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// LDS accessors (byte offsets into a __shared__ char array).
__device__ inline u32x4 lds_ld16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ inline void lds_st16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ inline void lds_st8(char* base, int off, u32x2 v) {
  *reinterpret_cast<u32x2*>(base + off) = v;
}
__device__ inline void lds_st4(char* base, int off, uint32_t v) {
  *reinterpret_cast<uint32_t*>(base + off) = v;
}

// Transposing LDS load (ds_read_b64_tr_b16). Within each group of 16 lanes, lane j
// receives 4 elements: element k is element (j % 4) of the 8 bytes addressed by lane
// 4*k + j/4 of the group. Lanes that address 4 consecutive rows x 4 consecutive 16-bit
// columns of a row-major tile thus gather a column slice (4 rows) per lane.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x2 lds_ld8_tr(const char* base, int off) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(base + off));
  return __builtin_bit_cast(u32x2, r);
}

// Register-class pins (empty asm, no instruction emitted): keep a value in the
// accumulation registers (AGPRs) or in the vector registers at this point. MFMA reads
// its operands and accumulator from either class; values only ever touched by MFMA are
// pinned to AGPRs so that kernels with more live state than 256 VGPRs do not shuttle
// them between the two register files every iteration.
__device__ inline void pin_agpr(f32x16& x) { asm volatile("" : "+a"(x)); }
__device__ inline void pin_agpr(u32x4& x) { asm volatile("" : "+a"(x)); }

// Byte permute: result byte k = byte sel_k of the 8-byte value {hi:lo}.
__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low 16-bit halves of two words, packed (a.lo | b.lo << 16); high halves likewise.
__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return perm(b, a, 0x05040100u); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

}  // namespace fa

namespace fa {

__device__ __host__ constexpr int align16(int x) { return (x + 15) & ~15; }

// Rows inside a 32-row block are relabelled in transposed LDS tiles so that the 8 rows
// one lane feeds to an MFMA step (rows 8*(t/4) + 4*h + t%4 + 16*s of the 32x32 result
// layout) sit in 8 consecutive slots: swap bits 2 and 3 of the row index.
__device__ constexpr int tr_pos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Reductions over the wave. Every lane ends with the same value; reading it back from
// the first lane tells the compiler so, and branches on it become scalar branches.
__device__ inline int wave_min(int v) {
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ inline int wave_max(int v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ inline float wave_fsum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ inline float wave_fmax(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
// Index of the calling wave inside its workgroup, as a wave-uniform (scalar) value.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------------
// Swizzled tiles filled by direct global -> LDS loads (global_load_lds_dwordx4).
// A tile of ROWS rows x D 16-bit elements is stored without padding (row = 2*D bytes);
// 16-byte chunk c of tile row r sits in chunk slot c ^ swz(r). With this permutation
// (a) 16-byte row reads by 16 lanes of 16 consecutive rows and (b) transposing 8-byte
// reads by 16 lanes of 4 consecutive rows x 32 bytes both touch 64 distinct LDS banks.
// swz depends on r mod 16 only.
// ---------------------------------------------------------------------------------
template <int D>
__device__ constexpr int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Scheduling fence: the compiler may not move instructions across it. Placed after a
// batch of LDS operand reads so the reads are all in flight before the MFMAs that use
// them (otherwise the scheduler interleaves them and each MFMA waits a full LDS latency).
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until at most N vector-memory operations of this wave are outstanding (direct
// LDS loads count here; they complete in issue order).
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Race-check build (compiled with FA_SYNC_CHECK=1 into a library of its own, which a test
// compares with the normal one): every ring step also waits for all of its loads and
// passes a full workgroup barrier right after issuing the next tile, so copies no longer
// overlap compute and no wave runs ahead of another. The normal build must give the
// same bits; a difference means an access that depends on timing.
#ifndef FA_SYNC_CHECK
#define FA_SYNC_CHECK 0
#endif
__device__ inline void sync_check() {
  if constexpr (FA_SYNC_CHECK != 0) {
    wait_vmem<0>();
    __syncthreads();
  }
}

// A read-and-wait LDS load written as inline assembly, for small tables that are filled
// before a loop and only read inside it. Written through the builtin path, such a read
// looks to the compiler as if it could alias the ring stages being filled by direct
// loads, and it puts a wait for every load in flight in front of it. The wait for the
// read itself is part of the same statement (the whole LDS queue is drained: use where
// no other LDS read is outstanding).
__device__ inline uint32_t lds_read_b32_now(const void* p) {
  const uint32_t a = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

// ---------------------------------------------------------------------------------
// Block-sparse tile lists. A workgroup walks tiles t_lo .. t_hi-1 along one axis; with a
// block bitmap some of them are needed by no wave. Each wave marks the tiles it needs in
// 64-tile words (need[wid][2c], need[wid][2c+1]: tiles t_lo + 64c + 0..31, 32..63); wave
// 0 then writes the tiles some wave needs, in order, to `list` as
//   entry = tile | (bit w set when wave w needs the tile) << 16
// and the list length to *n_s. Every thread of the workgroup calls this (two workgroup
// barriers); need_fn(t) is the calling lane's answer for tile t (only called for
// t < t_hi). Tiles must be below 65536. Returns the list length.
// ---------------------------------------------------------------------------------
template <int NW, int W2, typename NeedFn>
__device__ inline int build_tile_list(uint32_t (&need)[NW][W2], uint32_t* list, int* n_s,
                                      int wid, int lane, int t_lo, int t_hi, NeedFn need_fn) {
  static_assert(NW <= 16, "wave masks take the upper 16 bits of an entry");
  for (int c = 0; c * 64 < t_hi - t_lo; ++c) {
    const int t = t_lo + c * 64 + lane;
    const bool nd = t < t_hi && need_fn(t);
    const uint64_t m = __builtin_amdgcn_ballot_w64(nd);
    if (lane == 0) {
      need[wid][2 * c] = (uint32_t)m;
      need[wid][2 * c + 1] = (uint32_t)(m >> 32);
    }
  }
  __syncthreads();
  if (wid == 0) {
    int cnt = 0;
    for (int c = 0; c * 64 < t_hi - t_lo; ++c) {
      uint32_t lo = 0, hi = 0, waves = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t wl = need[w][2 * c], wh = need[w][2 * c + 1];
        lo |= wl;
        hi |= wh;
        waves |= (lane < 32 ? (wl >> lane) & 1u : (wh >> (lane - 32)) & 1u) << w;
      }
      const int before = (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
      if (waves != 0) list[cnt + before] = (uint32_t)(t_lo + c * 64 + lane) | (waves << 16);
      cnt += __builtin_popcount(lo) + __builtin_popcount(hi);
    }
    if (lane == 0) *n_s = cnt;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*n_s);
}

// Reads a list built by build_tile_list by position, with no LDS round trip per
// position: entries base .. base+63 and base+64 .. base+127 sit one per lane in two
// registers and come out through a lane read. slide(p) moves the window on by 64 once
// position p has left its first half (one LDS read per 64 positions), so after
// slide(p), at(q) is valid for p <= q < p + 64. CAP is the list's capacity.
template <int CAP>
struct ListWindow {
  const uint32_t* list;
  uint32_t w0, w1;
  int base, lane;
  __device__ void init(const uint32_t* l, int ln) {
    list = l;
    lane = ln;
    base = 0;
    w0 = lds_read_b32_now(&l[min(ln, CAP - 1)]);
    w1 = lds_read_b32_now(&l[min(64 + ln, CAP - 1)]);
  }
  __device__ uint32_t at(int p) const {
    const int r = p - base;
    return (uint32_t)(r < 64 ? __builtin_amdgcn_readlane((int)w0, r)
                             : __builtin_amdgcn_readlane((int)w1, r - 64));
  }
  __device__ void slide(int p) {
    if (p - base >= 64) {
      base += 64;
      w0 = w1;
      w1 = lds_read_b32_now(&list[min(base + 64 + lane, CAP - 1)]);
    }
  }
};

// ---------------------------------------------------------------------------------
// Direct global -> LDS loads, in two forms.
//  * buffer form (buffer_load_dword{,x4} ... lds): a resource covers the bytes from a
//    wave-uniform base; per-lane offsets are 32-bit (every caller keeps them inside one
//    matrix of fewer than 2^32 bytes), the range check is off (num_records = 0xffffffff)
//    and word 3 selects 32-bit raw data. The compiler tracks it with the vector-memory
//    counter only.
//  * global form (global_load_lds_dword{,x4}): a FLAT-encoded instruction that writes
//    LDS. While one is in flight the compiler counts LDS reads as possibly out of order
//    and waits for every one of them (lgkmcnt(0)) before using any.
// The forward and dQ passes use the buffer form (their MFMAs then wait only for their own
// operands: 512 -> 520 us and 734 -> 742 us measured the other way on the bf16 causal
// B2 H16 N8192 d128 shape); the dK/dV pass measured faster with the global form (1187
// against 1229 us), so each kernel picks its form (BUF).
// ---------------------------------------------------------------------------------
template <bool BUF>
struct DmaBase;
template <>
struct DmaBase<true> {
  __amdgpu_buffer_rsrc_t r;
  __device__ explicit DmaBase(const void* base)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffffu,
                                            0x00020000)) {}
  // one wave-wide direct load of SIZE (4 or 16) bytes per lane from byte offset `voff`:
  // lane i fills bytes [SIZE*i, SIZE*i + SIZE) of the window at `lds` (wave-uniform)
  template <int SIZE>
  __device__ void load(uint32_t voff, char* lds) const {
    static_assert(SIZE == 4 || SIZE == 16, "4 or 16 bytes per lane");
    auto* l = (__attribute__((address_space(3))) void*)lds;
    if constexpr (SIZE == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff, 0, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 4, voff, 0, 0, 0);
  }
};
template <>
struct DmaBase<false> {
  const char* p;
  __device__ explicit DmaBase(const void* base) : p(static_cast<const char*>(base)) {}
  template <int SIZE>
  __device__ void load(uint32_t voff, char* lds) const {
    static_assert(SIZE == 4 || SIZE == 16, "4 or 16 bytes per lane");
    auto* l = (__attribute__((address_space(3))) void*)lds;
    if constexpr (SIZE == 16) __builtin_amdgcn_global_load_lds(p + voff, l, 16, 0, 0);
    else __builtin_amdgcn_global_load_lds(p + voff, l, 4, 0, 0);
  }
};
// 4 bytes per lane from element `idx` of the float array at the wave-uniform `base`
template <bool BUF>
__device__ inline void dma4(const float* base, uint32_t idx, char* lds) {
  DmaBase<BUF>(base).template load<4>(idx * 4u, lds);
}

// One wave-wide direct load moves 1 KB: lane i fills bytes [16i, 16i+16) of the window
// (the LDS address comes from the wave-uniform window base). A tile is kOps windows,
// split evenly over the NW waves of the workgroup.
template <int ROWS, int D, int NW>
struct DmaTile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kBytes = ROWS * kRowBytes;
  static constexpr int kChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kRowsPerOp = 1024 / kRowBytes;  // rows one window holds
  static constexpr int kOps = kBytes / 1024;
  static constexpr int kOpsPerWave = kOps / NW;
  static_assert(kOpsPerWave >= 1 && kOpsPerWave * NW == kOps, "tile split over waves");

  int row[kOpsPerWave];  // tile-local row this lane loads, per window
  int col[kOpsPerWave];  // byte offset of its chunk inside the global row

  __device__ inline void init(int wid, int lane) {
#pragma unroll
    for (int j = 0; j < kOpsPerWave; ++j) {
      const int u = wid * kOpsPerWave + j;
      row[j] = u * kRowsPerOp + lane / kChunks;
      col[j] = 16 * ((lane % kChunks) ^ swz<D>(row[j]));  // slot lane%kChunks holds this chunk
    }
  }
  // this wave's share of rows [row0, row0 + ROWS) of a row-major (nrows x D) matrix;
  // rows past the end repeat the last row (their scores are masked). The byte offset
  // inside the matrix is formed in 32 bits (a matrix of one (b, h) holds fewer than 2^32
  // bytes: N * d <= INT_MAX elements of 2 bytes), so the load takes the wave-uniform base
  // plus a 32-bit per-lane offset and no 64-bit address per lane stays live in a loop.
  template <bool BUF = true, typename T>
  __device__ inline void load(const T* base, int row0, int nrows, char* lds, int wid) const {
    const DmaBase<BUF> rs(base);
#pragma unroll
    for (int j = 0; j < kOpsPerWave; ++j) {
      const uint32_t r = (uint32_t)min(row0 + row[j], nrows - 1);
      const uint32_t off = r * (uint32_t)kRowBytes + (uint32_t)col[j];
      rs.template load<16>(off, lds + (wid * kOpsPerWave + j) * 1024);
    }
  }
};

// float32 bias tiles carried by the same direct-load rings as K and V (4-byte loads, so
// any row stride, broadcast stride and ragged key count works: every lane's element index
// is clamped into the matrix, and clamped entries are masked by the kernel).
//
// Query-on-lane kernels (scores S^T: lane = query row n of the wave, registers = keys):
// the wave's 32 rows x BC keys, row-major; one direct load fills a 64-float window of
// 64/BC rows, and windows are 272 bytes apart, so that the 16-byte reads of 4 keys by
// lanes of consecutive rows fall into distinct bank groups.
template <int BC>
struct BiasRowTile {
  static_assert(BC == 32 || BC == 64, "key tile");
  static constexpr int kRW = 64 / BC;        // rows per window
  static constexpr int kWin = 272;           // bytes between windows
  static constexpr int kOps = 32 / kRW;      // direct loads per wave per tile
  static constexpr int kWaveBytes = kOps * kWin;
  // rows [wq0, wq0 + 32) (clamped to nq - 1), keys [kt0, kt0 + BC) (clamped to nk - 1) of
  // the (b, h) matrix at `base` with row stride si, into this wave's region `lds`
  __device__ static inline void load(const float* base, long long si, int wq0, int nq, int kt0,
                                     int nk, char* lds, int lane) {
    // the resource starts at the tile's first row, so offsets stay within 32 rows
    const int r0 = min(wq0, nq - 1);
    const DmaBase<true> rs(base + (long long)r0 * si);
    const uint32_t j = (uint32_t)min(kt0 + lane % BC, nk - 1);
#pragma unroll
    for (int w = 0; w < kOps; ++w) {
      const uint32_t i = (uint32_t)(min(wq0 + w * kRW + lane / BC, nq - 1) - r0);
      rs.load<4>((i * (uint32_t)si + j) * 4u, lds + w * kWin);
    }
  }
  // keys c0 .. c0 + 3 (c0 a multiple of 4) of wave row r
  __device__ static inline f32x4 read(const char* lds, int r, int c0) {
    return *reinterpret_cast<const f32x4*>(lds + (r / kRW) * kWin + ((r % kRW) * BC + c0) * 4);
  }
};

// Key-on-lane kernel (dK/dV: scores S; lane l holds key l % 32 of the wave's 32 keys, and
// the 16 registers of a 32-query block rows res_row(g, l / 32)): the 64-row query tile x the
// wave's 32 keys, stored in the order the lanes read it: window (qb, g) holds at lane l
// the entry of row 32 qb + res_row(g, l / 32) and key l % 32, so a read is one 4-byte
// access per lane with no bank conflict, and each direct load reads two 128-byte row
// segments.
struct BiasColTile {
  static constexpr int kOps = 32;            // windows (2 query blocks x 16 registers)
  static constexpr int kWaveBytes = kOps * 256;
  __device__ static inline void load(const float* base, long long si, int q0t, int nq, int kw0,
                                     int nk, char* lds, int lane) {
    // the resource starts at the tile's first row, so offsets stay within 64 rows
    const int r0 = min(q0t, nq - 1);
    const DmaBase<false> rs(base + (long long)r0 * si);  // (dK/dV pass: global form)
    const uint32_t j = (uint32_t)min(kw0 + (lane & 31), nk - 1);
    const int hh = lane >> 5;
#pragma unroll
    for (int w = 0; w < kOps; ++w) {
      const int qb = w >> 4, g = w & 15;
      const uint32_t i =
          (uint32_t)(min(q0t + 32 * qb + 8 * (g >> 2) + 4 * hh + (g & 3), nq - 1) - r0);
      rs.load<4>((i * (uint32_t)si + j) * 4u, lds + w * 256);
    }
  }
  __device__ static inline float read(const char* lds, int qb, int g, int lane) {
    return *reinterpret_cast<const float*>(lds + (qb * 16 + g) * 256 + lane * 4);
  }
};

// A [ROWS x D] tile of 16-bit elements copied global -> registers -> LDS by NT threads.
// Thread b owns KQ consecutive rows of one 16-byte column chunk, so the same registers
// can be written row-major ("natural": row stride NSTRIDE bytes) and transposed
// ("T": D rows of ROWS slots, row stride TSTRIDE bytes, 16-byte chunks XOR-swizzled by
// (row/16), slot of row r = tr_pos(r)). Global reads of a warp cover whole rows.
template <int ROWS, int D, int NT>
struct TileCopy {
  static constexpr int kRowChunks = D / 8;
  static constexpr int kRaw = ROWS * kRowChunks / NT;
  static constexpr int KQ = kRaw >= 4 ? 4 : kRaw;
  static constexpr int kGroups = KQ > 0 ? kRaw / KQ : 0;
  static constexpr int kTChunks = ROWS / 8;
  static_assert(KQ >= 2 && kGroups * KQ * NT == ROWS * kRowChunks, "tile copy split");

  u32x4 r[kGroups][KQ];

  template <typename T>
  __device__ inline void load(const T* base, int row0, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const int b = tid + i * NT;
      const int grp = b / kRowChunks, col = b % kRowChunks;
#pragma unroll
      for (int e = 0; e < KQ; ++e) {
        const int row = min(row0 + grp * KQ + e, nrows - 1);  // rows past the end: masked
        r[i][e] = ldg16(base + (size_t)row * D + col * 8);
      }
    }
  }

  template <int NSTRIDE>
  __device__ inline void store_natural(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const int b = tid + i * NT;
      const int grp = b / kRowChunks, col = b % kRowChunks;
#pragma unroll
      for (int e = 0; e < KQ; ++e) lds_st16(lds, (grp * KQ + e) * NSTRIDE + col * 16, r[i][e]);
    }
  }

  template <int TSTRIDE>
  __device__ static inline int t_off(int row, int chunk) {
    return row * TSTRIDE + 16 * (chunk ^ ((row >> 4) & (kTChunks - 1)));
  }

  template <int TSTRIDE>
  __device__ inline void store_T(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
      const int b = tid + i * NT;
      const int grp = b / kRowChunks, col = b % kRowChunks;
      const int pos = tr_pos(grp * KQ);  // KQ consecutive rows -> KQ consecutive slots
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int row = col * 8 + dd;
        const int w = dd >> 1;
        const int byte = t_off<TSTRIDE>(row, pos >> 3) + (pos & 7) * 2;
        if constexpr (KQ == 4) {
          u32x2 val;
          val[0] = (dd & 1) ? pack_hi(r[i][0][w], r[i][1][w]) : pack_lo(r[i][0][w], r[i][1][w]);
          val[1] = (dd & 1) ? pack_hi(r[i][2][w], r[i][3][w]) : pack_lo(r[i][2][w], r[i][3][w]);
          lds_st8(lds, byte, val);
        } else {
          lds_st4(lds, byte, (dd & 1) ? pack_hi(r[i][0][w], r[i][1][w]) : pack_lo(r[i][0][w], r[i][1][w]));
        }
      }
    }
  }
};

// Workgroup -> (bh, block along the kernel's parallel axis), heaviest block first.
// With kSchedXcd every (b, h) stays on one of the 8 XCDs (blocks are dealt to XCDs
// round-robin), so its K/V (or Q/dO) is shared through that XCD's L2; the blocks of one
// head come out heaviest first, head after head. kSchedXcdLpt keeps the heads on their
// XCDs but orders the blocks of all the XCD's heads by weight (every head's heaviest
// block first, then the next): the longest-first order over the XCD's slots, so that the
// last blocks to start are the shortest. On the bf16 causal B4 H16 N2048 d128 forward
// 95.6-103.5 -> 77.5-78.5 us, on B2 H16 N8192 d128 forward 502-507 -> 487-492 us, dK/dV
// 1180-1351 -> 1165-1318 us, dQ 727-780 -> 696-724 us (interleaved on one box).
__device__ inline void map_block(int L, int BH, int nblk, int sched, bool reverse, int& bh, int& blk) {
  int s;
  if (sched == 2) {
    // heads pinned to XCDs as above, blocks ordered by weight across the XCD's heads
    // (all heads' heaviest blocks first): the longest-first order over the XCD's slots
    const int x = L & 7, hx = BH >> 3;
    s = L >> 3;
    bh = x + 8 * (s % hx);
    const int r = s / hx;
    blk = reverse ? nblk - 1 - r : r;
    return;
  }
  if (sched == 1) {
    const int x = L & 7;
    s = L >> 3;
    bh = x + 8 * (s / nblk);
  } else {
    s = L;
    bh = L / nblk;
  }
  const int r = s % nblk;
  blk = reverse ? nblk - 1 - r : r;
}

}  // namespace fa
