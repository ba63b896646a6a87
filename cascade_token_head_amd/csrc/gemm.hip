// Q/K/V and output projections of the kept heads (SpAtten, section II
// "Attention mechanism": inputs split into per-head Q, K, V; head outputs
// concatenated; "Cascade pruning": a pruned head's Q/K/V chunks are gone).
//
// bf16 path: 128x128x64 workgroup tiles of four 64x64 waves, or for large
// projections 256x256x64 tiles of eight 128x64 waves, on gfx950 MFMA
// 32x32x16 (fp32 accumulate), operands staged through swizzled LDS rows
// with double buffering. Head pruning is a gather: each output
// column block (QKV) or K block (output projection) reads the weight rows
// or columns of the head kept in that slot, per sequence. When every head
// is kept all sequences share the weights and M tiles run across sequence
// boundaries; otherwise M tiles stay inside one sequence.
// fp32 path: a plain 64x64 VALU tile for the fp32 workload.
#include "common.hpp"
#include "importance.hpp"
#include "kernels.hpp"
#include "timing.hpp"

#include <cmath>

namespace spatten {
namespace {

enum { kQkvPrefill = 0, kQkvDecode = 1, kOut = 2 };

struct GemmParams {
  const void* A;
  int64_t lda;
  const void* W0;
  const void* W1;
  const void* W2;
  int64_t ldw;
  const int32_t* head_idx;
  int batch, n, seq_tiled, mt_per_seq, M_total, N, K;
  int tiles_y;  // M tiles of the tiled kernel (set by its launcher)
  int h_kept, dh, D, n_pad;
  void* out0;
  void* out1;
  void* out2;
  int64_t kv_bs;
  // skinny path: workgroups [0, gemm_blocks) project; the rest run the
  // decode importance pass (imp.pending)
  int gemm_blocks;
  ImpArgs imp;
};

// Row of M tile `mt_flat`, local row r -> (valid, sequence, row in sequence)
struct RowMap {
  bool valid;
  int b, m;
};

__device__ __forceinline__ RowMap map_row(const GemmParams& p, int tile_y, int r, int BM) {
  RowMap rm;
  if (p.seq_tiled) {
    rm.b = tile_y / p.mt_per_seq;
    rm.m = (tile_y - rm.b * p.mt_per_seq) * BM + r;
    rm.valid = rm.m < p.n;
  } else {
    const int g = tile_y * BM + r;
    rm.valid = g < p.M_total;
    rm.b = g / p.n;
    rm.m = g - rm.b * p.n;
  }
  return rm;
}

__device__ __forceinline__ int head_of(const GemmParams& p, int b, int s) {
  return p.seq_tiled ? p.head_idx[b * p.h_kept + s] : s;
}

// Weight row (QKV) for output column ncol of sequence b.
template <typename T>
__device__ __forceinline__ const T* qkv_weight_row(const GemmParams& p, int b, int ncol) {
  const int hd = p.h_kept * p.dh;
  const int which = ncol / hd;
  const int rem = ncol - which * hd;
  const int s = rem / p.dh, c = rem - s * p.dh;
  const void* W = which == 0 ? p.W0 : (which == 1 ? p.W1 : p.W2);
  return static_cast<const T*>(W) + int64_t(head_of(p, b, s) * p.dh + c) * p.ldw;
}

template <typename T, int MODE>
__device__ __forceinline__ void store_out(const GemmParams& p, const RowMap& rm, int ncol,
                                          float v) {
  if (MODE == kOut) {
    const int64_t i = (int64_t(rm.b) * p.n + rm.m) * p.D + ncol;
    store_elem<T>(p.out0, i, load_elem<T>(p.out0, i) + v);
    return;
  }
  const int hd = p.h_kept * p.dh;
  const int which = ncol / hd;
  const int rem = ncol - which * hd;
  const int s = rem / p.dh, c = rem - s * p.dh;
  if (MODE == kQkvDecode) {
    if (which == 0)
      store_elem<T>(p.out0, int64_t(rm.b) * p.D + rem, v);
    else
      store_elem<T>(which == 1 ? p.out1 : p.out2, int64_t(rm.b) * p.kv_bs + rem, v);
    return;
  }
  const int64_t bs = int64_t(rm.b) * p.h_kept + s;
  if (which < 2)
    store_elem<T>(which == 0 ? p.out0 : p.out1, (bs * p.n_pad + rm.m) * p.dh + c, v);
  else
    store_elem<T>(p.out2, (bs * p.dh + c) * p.n_pad + rm.m, v);
}

// ------------------------------------------------------------------ bf16 MFMA

constexpr int BM = 128, BN = 128, BK = 64, LDS_K = BK + 8;

template <int MODE>
__global__ void __launch_bounds__(256)
gemm_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDS_K];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDS_K];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile_y = blockIdx.y, n0 = blockIdx.x * BN;
  const int b_tile = p.seq_tiled ? tile_y / p.mt_per_seq : 0;

  // global -> LDS assignment: 4 chunks of 16 B per thread for each operand
  const bf16_t* a_src[4];
  const bf16_t* w_src[4];
  int ld_row[4];
  const int kc = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    ld_row[i] = r;
    RowMap rm = map_row(p, tile_y, r, BM);
    if (!rm.valid) {  // clamp to a real row; its results are never stored
      rm = p.seq_tiled ? RowMap{true, rm.b, p.n - 1} : RowMap{true, p.batch - 1, p.n - 1};
    }
    a_src[i] = static_cast<const bf16_t*>(p.A) + (int64_t(rm.b) * p.n + rm.m) * p.lda + kc;
    int ncol = n0 + r;
    if (ncol >= p.N) ncol = p.N - 1;
    if (MODE == kOut)
      w_src[i] = static_cast<const bf16_t*>(p.W0) + int64_t(ncol) * p.ldw;
    else
      w_src[i] = qkv_weight_row<bf16_t>(p, b_tile, ncol) + kc;
  }

  const int KT = p.K / BK;
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    int wcol = k0;
    if (MODE == kOut) {
      const int s = k0 / p.dh;
      wcol = head_of(p, b_tile, s) * p.dh + (k0 - s * p.dh) + kc;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
      rb[i] = *reinterpret_cast<const u32x4*>(MODE == kOut ? w_src[i] + wcol : w_src[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][ld_row[i] * LDS_K + kc]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][ld_row[i] * LDS_K + kc]) = rb[i];
    }
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int fr = lane & 31, fk = (lane >> 5) * 8;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &As[buf][(wm + 32 * i + fr) * LDS_K + kk + fk]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &Bs[buf][(wn + 32 * j + fr) * LDS_K + kk + fk]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const RowMap rm = map_row(p, tile_y, lr, BM);
      if (!rm.valid) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ncol = n0 + wn + 32 * j + fr;
        if (ncol < p.N) store_out<bf16_t, MODE>(p, rm, ncol, acc[i][j][r]);
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA, large tiles
//
// BM x BN x 64 workgroup tiles, four waves in a 2 x 2 grid, each wave
// (BM/2) x (BN/2) with 32x32x16 MFMAs, so every LDS fragment feeds BN/64
// or BM/64 MFMAs. LDS rows are 128 bytes with the 16-byte chunks XOR-
// swizzled by the row index: the eight rows a group of lanes reads at one
// k offset land in different bank groups without padding, and two
// stages of a 256 x 256 tile fit in 128 KB. Epilogue index math is hoisted:
// column terms once per MFMA column tile, row terms advanced incrementally.

// pimp (output projection): workgroups past the tiles run the prefill
// importance pass when pimp.pending; the grid then holds its workgroups.
template <int MODE, int BM, int BN, int NW>
__global__ void __launch_bounds__(64 * NW, (BM * BN <= 128 * 128) ? 2 : 1)
gemm_tile_kernel(GemmParams p, PrefillImp pimp) {
  constexpr int BKT = 64;
  constexpr int NT = 64 * NW;                 // threads
  constexpr int WGN = NW == 8 ? 4 : 2;        // waves across N (2 or 4) x 2 across M
  constexpr int WM = BM / 2, WN = BN / WGN, TI = WM / 32, TJ = WN / 32;
  constexpr int NA = BM * 8 / NT, NB = BN * 8 / NT;  // 16-byte chunks per thread
  constexpr int RS = NT / 8;                  // rows between a thread's chunks
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * BKT];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * BKT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroup i runs on XCD i % 8, and each XCD takes one contiguous run of
  // a grouped tile order: groups of GM row tiles, swept column by column.
  // The ~64 tiles an XCD holds at once then span GM row blocks of A and
  // 64 / GM weight tiles, which fit its 4 MB L2 together.
  constexpr int GM = 8;
  const int ntx = int(ceil_div(p.N, BN));
  const int total = ntx * p.tiles_y;
  const int per_xcd = int(ceil_div(total, 8));
  if (MODE == kOut && int(blockIdx.x) >= 8 * per_xcd) {
    // dispatched after every tile, so they run beside the last round
    prefill_importance_block(pimp, int(blockIdx.x) - 8 * per_xcd);
    return;
  }
  const int t = (int(blockIdx.x) & 7) * per_xcd + (int(blockIdx.x) >> 3);
  if (t >= total) return;
  const int grp = t / (GM * ntx), in_grp = t - grp * (GM * ntx);
  const int rows_g = min(GM, p.tiles_y - grp * GM);
  const int tile_y = grp * GM + in_grp % rows_g, n0 = (in_grp / rows_g) * BN;
  const int b_tile = p.seq_tiled ? tile_y / p.mt_per_seq : 0;
  const int kc = tid & 7;  // 16-byte chunk along k this thread loads

  const bf16_t* a_src[NA];
  const bf16_t* w_src[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = (tid >> 3) + RS * i;
    RowMap rm = map_row(p, tile_y, r, BM);
    if (!rm.valid) rm = p.seq_tiled ? RowMap{true, rm.b, p.n - 1} : RowMap{true, p.batch - 1, p.n - 1};
    a_src[i] = static_cast<const bf16_t*>(p.A) + (int64_t(rm.b) * p.n + rm.m) * p.lda + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = (tid >> 3) + RS * i;
    int ncol = n0 + r;
    if (ncol >= p.N) ncol = p.N - 1;
    if (MODE == kOut)
      w_src[i] = static_cast<const bf16_t*>(p.W0) + int64_t(ncol) * p.ldw + kc * 8;
    else
      w_src[i] = qkv_weight_row<bf16_t>(p, b_tile, ncol) + kc * 8;
  }
  // LDS rows are 128 bytes; gfx950 serves 16 lanes of a b128 access from 64
  // banks, i.e. two rows per cycle, so chunk slots are XOR-swizzled by
  // (row >> 1) & 7: the 16 rows a half-wave reads at one k offset then hit
  // 16 distinct 16-byte bank groups. Slot of this thread's chunk in row r:
  // r*64 + ((kc ^ ((r >> 1) & 7)) * 8).
  const int st_off = (((tid >> 4) & 7) ^ kc) * 8 + (tid >> 3) * BKT;

  const int KT = p.K / BKT;
  // two register staging sets: the tile stored into LDS at the start of
  // iteration kt was requested two iterations earlier
  u32x4 ra0[NA], rb0[NB], ra1[NW == 4 ? NA : 1], rb1[NW == 4 ? NB : 1];
  auto gload = [&](u32x4* ra, u32x4* rb, int kt) {
    const int k0 = kt * BKT;
    int wk = k0;
    if (MODE == kOut) {
      const int s = k0 / p.dh;
      wk = head_of(p, b_tile, s) * p.dh + (k0 - s * p.dh);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < NB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(w_src[i] + wk);
  };
  auto sstore = [&](const u32x4* ra, const u32x4* rb, int buf) {
    // rows tid/8 + RS i keep the same (row >> 1) & 7, so one swizzled offset serves all i
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][st_off + RS * i * BKT]) = ra[i];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      *reinterpret_cast<u32x4*>(&Bs[buf][st_off + RS * i * BKT]) = rb[i];
  };

  floatx16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = (wave / WGN) * WM, wn = (wave % WGN) * WN;
  const int fr = lane & 31, G = lane >> 5;
  // fragment rows wm + 32 i + fr all share (row >> 1) & 7 == (fr >> 1) & 7
  const int fsw = (fr >> 1) & 7;

  auto compute = [&](int buf) {
    bf16x8 af[2][TI], bfr[2][TJ];
    auto frag = [&](int kk, int slot) {
      const int ch = ((2 * kk + G) ^ fsw) * 8;
#pragma unroll
      for (int i = 0; i < TI; ++i)
        af[slot][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(&As[buf][(wm + 32 * i + fr) * BKT + ch]));
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bfr[slot][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&Bs[buf][(wn + 32 * j + fr) * BKT + ch]));
    };
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) frag(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = mfma32x32x16(af[kk & 1][i], bfr[kk & 1][j], acc[i][j]);
    }
    // keep that order through scheduling: reads of slice 0, then per slice
    // the next slice's reads ahead of this slice's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, TI + TJ, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, TI + TJ, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ, 0);
    }
  };

  gload(ra0, rb0, 0);
  sstore(ra0, rb0, 0);
  if (KT > 1) gload(ra0, rb0, 1);
  if constexpr (NW == 4) {
    if (KT > 2) gload(ra1, rb1, 2);
  }
  __syncthreads();
  // Pairs of steps with no exit between them, so the accumulators stay in
  // place across the loop back-edge. Four waves keep two register staging
  // sets (loads two tiles ahead); eight waves, with twice the accumulators
  // per wave, keep one (one tile ahead).
  for (int kt = 0; kt + 1 < KT; kt += 2) {
    if constexpr (NW == 4) {
      // even step: compute tile kt from buffer 0, stage tile kt+1 into buffer 1
      sstore(ra0, rb0, 1);
      if (kt + 3 < KT) gload(ra0, rb0, kt + 3);
      compute(0);
      __syncthreads();
      // odd step: compute tile kt+1 from buffer 1, stage tile kt+2 into buffer 0
      if (kt + 2 < KT) sstore(ra1, rb1, 0);
      if (kt + 4 < KT) gload(ra1, rb1, kt + 4);
      compute(1);
      __syncthreads();
    } else {
      sstore(ra0, rb0, 1);
      if (kt + 2 < KT) gload(ra0, rb0, kt + 2);
      compute(0);
      __syncthreads();
      if (kt + 2 < KT) sstore(ra0, rb0, 0);
      if (kt + 3 < KT) gload(ra0, rb0, kt + 3);
      compute(1);
      __syncthreads();
    }
  }
  if (KT & 1) {  // the last (even) tile, staged by the final odd step
    compute(0);
    __syncthreads();  // the epilogue stage reuses As
  }

  // ---- epilogue: each 32 x 32 MFMA block goes through a 2 KB per-wave LDS
  // stage (row-major, or transposed for V^T) and leaves as 16-byte stores.
  const int hd = p.h_kept * p.dh;
  const float inv_n = 1.0f / float(p.n);
  // stage rows are padded to 40 elements (80 bytes): the transposed writes
  // of one store instruction then spread over 16 bank groups
  constexpr int SS = 40;
  bf16_t* stage = &As[0][0] + wave * (32 * SS);
  auto row_of = [&](int lr, int& b, int& m) -> bool {
    if (p.seq_tiled) {
      b = b_tile;
      m = (tile_y - b_tile * p.mt_per_seq) * BM + lr;
      return m < p.n;
    }
    const int g = tile_y * BM + lr;
    b = int(float(g) * inv_n);
    if (b * p.n > g) --b;
    if ((b + 1) * p.n <= g) ++b;
    m = g - b * p.n;
    return g < p.M_total;
  };
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int c0 = n0 + wn + 32 * j;  // first column of this block (uniform)
    if (c0 >= p.N) continue;
    const int which = MODE == kOut ? 0 : c0 / hd;
    const bool trans = MODE == kQkvPrefill && which == 2;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r0 = wm + 32 * i;  // first local row of this block
      if (trans) {
        // registers 4q .. 4q+3 are rows 8q + 4G .. +3 of column fr: one
        // 8-byte write each
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint64_t pk = uint64_t(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1])) |
                              (uint64_t(pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])) << 32);
          *reinterpret_cast<uint64_t*>(&stage[fr * SS + 8 * q + 4 * G]) = pk;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = 8 * (r >> 2) + 4 * G + (r & 3);
          stage[rr * SS + fr] = f32_to_bf16(acc[i][j][r]);
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ch = lane + 64 * q;        // 128 chunks of 8 elements
        const int a8 = ch >> 2, o8 = (ch & 3) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(&stage[a8 * SS + o8]);
        if (!trans) {
          // a8 = row in block, o8 = column offset
          int b, m;
          if (!row_of(r0 + a8, b, m)) continue;
          const int col = c0 + o8;
          if (MODE == kOut) {
            bf16_t* x = static_cast<bf16_t*>(p.out0) + (int64_t(b) * p.n + m) * p.D + col;
            u32x4 xv = *reinterpret_cast<const u32x4*>(x);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lo = __uint_as_float(xv[e] << 16) + __uint_as_float(v[e] << 16);
              const float hi = __uint_as_float(xv[e] & 0xffff0000u) +
                               __uint_as_float(v[e] & 0xffff0000u);
              xv[e] = pack_bf16x2(lo, hi);
            }
            *reinterpret_cast<u32x4*>(x) = xv;
          } else {
            const int rem = col - which * hd;
            const int s_ = rem / p.dh, cc = rem - s_ * p.dh;
            bf16_t* d = static_cast<bf16_t*>(which == 0 ? p.out0 : p.out1) +
                        ((int64_t(b) * p.h_kept + s_) * p.n_pad + m) * p.dh + cc;
            *reinterpret_cast<u32x4*>(d) = v;
          }
        } else {
          // a8 = column in block, o8 = first of 8 consecutive rows
          const int col = c0 + a8;
          const int rem = col - 2 * hd;
          const int s_ = rem / p.dh, cc = rem - s_ * p.dh;
          int b, m, b7, m7;
          const bool v0 = row_of(r0 + o8, b, m);
          const bool v7 = row_of(r0 + o8 + 7, b7, m7);
          bf16_t* base = static_cast<bf16_t*>(p.out2);
          if (v0 && v7 && b7 == b && (m & 7) == 0) {
            *reinterpret_cast<u32x4*>(base + ((int64_t(b) * p.h_kept + s_) * p.dh + cc) * p.n_pad + m) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              int be, me;
              if (!row_of(r0 + o8 + e, be, me)) continue;
              const uint32_t w32 = v[e >> 1];
              base[((int64_t(be) * p.h_kept + s_) * p.dh + cc) * p.n_pad + me] =
                  bf16_t((e & 1) ? (w32 >> 16) : (w32 & 0xffffu));
            }
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ------------------------------------------------------------------ decode projections
//
// M = batch rows (at most 64): the weights are the traffic. A workgroup owns
// 16 output columns of one 16-row tile (the tiles of one column block read
// the same weights, from one XCD's L2 when the column-block count is a
// multiple of 8); its waves split K into KT 32-wide steps each and issue
// every fragment load (a weight row's and the tile's 8 consecutive k per
// lane) before the first 16x16x32 MFMA. Partial sums meet in LDS, in wave
// order. The output projection's residual is requested at the start.

constexpr int kSkinnyMaxWaves = 8;

template <int MODE, int KT>
__global__ void __launch_bounds__(64 * kSkinnyMaxWaves)
gemm_skinny_kernel(GemmParams p) {
  if (int(blockIdx.x) >= p.gemm_blocks) {
    importance_block(p.imp, int(blockIdx.x) - p.gemm_blocks);
    return;
  }
  __shared__ floatx4 part[kSkinnyMaxWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int ntiles = p.N >> 4;
  const int rt = int(blockIdx.x) / ntiles, n0 = (int(blockIdx.x) - rt * ntiles) * 16;
  const int l16 = lane & 15, kq = (lane >> 4) * 8;
  const int kbeg = wave * KT * 32 + kq;
  const int ncol = n0 + l16;
  // residual rows of this lane in the epilogue (wave 0)
  float res[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (MODE == kOut && wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = rt * 16 + 4 * (lane >> 4) + i;
      if (b < p.M_total) res[i] = bf16_to_f32(static_cast<const bf16_t*>(p.out0)[int64_t(b) * p.D + ncol]);
    }
  }
  const bf16_t* w_row = MODE == kOut
                            ? static_cast<const bf16_t*>(p.W0) + int64_t(ncol) * p.ldw + kbeg
                            : qkv_weight_row<bf16_t>(p, 0, ncol) + kbeg;
  int row = 16 * rt + l16;
  if (row >= p.M_total) row = p.M_total - 1;
  const bf16_t* a_row = static_cast<const bf16_t*>(p.A) + int64_t(row) * p.lda + kbeg;
  u32x4 bv[KT], av[KT];
#pragma unroll
  for (int u = 0; u < KT; ++u) bv[u] = *reinterpret_cast<const u32x4*>(w_row + 32 * u);
#pragma unroll
  for (int u = 0; u < KT; ++u) av[u] = *reinterpret_cast<const u32x4*>(a_row + 32 * u);
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < KT; ++u) acc = mfma16x16x32(as_bf16x8(av[u]), as_bf16x8(bv[u]), acc);
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nw; ++w) acc += part[w][lane];
  // C fragment: lane holds rows 4*(lane/16) + i of the tile, column l16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = rt * 16 + 4 * (lane >> 4) + i;
    if (b >= p.M_total) continue;
    const float v = acc[i];
    if (MODE == kOut) {
      static_cast<bf16_t*>(p.out0)[int64_t(b) * p.D + ncol] = f32_to_bf16(res[i] + v);
    } else {
      const int hd = p.h_kept * p.dh;
      const int which = ncol / hd;
      const int rem = ncol - which * hd;
      bf16_t* d = which == 0 ? static_cast<bf16_t*>(p.out0) + int64_t(b) * p.D
                             : static_cast<bf16_t*>(which == 1 ? p.out1 : p.out2) +
                                   int64_t(b) * p.kv_bs;
      d[rem] = f32_to_bf16(v);
    }
  }
}

// Smallest K step count per wave (1, 2, 4 or 8) that splits K over at most
// kSkinnyMaxWaves waves; 0 if none does.
inline int skinny_kt(int K) {
  if (K % 32 != 0) return 0;
  const int steps = K / 32;
  for (int kt = 1; kt <= 8; kt *= 2)
    if (steps % kt == 0 && steps / kt <= kSkinnyMaxWaves) return kt;
  return 0;
}

template <int MODE>
int run_skinny(GemmParams& p, int kt, hipStream_t stream, const char* name) {
  p.gemm_blocks = (p.N / 16) * int((p.M_total + 15) / 16);
  const int imp_blocks = p.imp.pending ? p.imp.batch * p.imp.pieces : 0;
  const dim3 grid(unsigned(p.gemm_blocks + imp_blocks));
  const int threads = 64 * (p.K / 32 / kt);
  switch (kt) {
    case 1: SPATTEN_TIMED(name, stream, gemm_skinny_kernel<MODE, 1><<<grid, threads, 0, stream>>>(p)); break;
    case 2: SPATTEN_TIMED(name, stream, gemm_skinny_kernel<MODE, 2><<<grid, threads, 0, stream>>>(p)); break;
    case 4: SPATTEN_TIMED(name, stream, gemm_skinny_kernel<MODE, 4><<<grid, threads, 0, stream>>>(p)); break;
    default: SPATTEN_TIMED(name, stream, gemm_skinny_kernel<MODE, 8><<<grid, threads, 0, stream>>>(p)); break;
  }
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

// ------------------------------------------------------------------ fp32 VALU

constexpr int FT = 64, FK = 16;

template <int MODE>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(GemmParams p) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  const int tid = threadIdx.x;
  const int tile_y = blockIdx.y, n0 = blockIdx.x * FT;
  const int b_tile = p.seq_tiled ? tile_y / p.mt_per_seq : 0;
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  float acc[4][4] = {};
  // loader: 64 rows x 16 k per operand, 4 elements per thread
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  RowMap rm = map_row(p, tile_y, lr, FT);
  if (!rm.valid) rm = p.seq_tiled ? RowMap{true, rm.b, p.n - 1} : RowMap{true, p.batch - 1, p.n - 1};
  const float* a_row = static_cast<const float*>(p.A) + (int64_t(rm.b) * p.n + rm.m) * p.lda;
  int ncol = n0 + lr;
  if (ncol >= p.N) ncol = p.N - 1;
  const float* w_row = MODE == kOut ? static_cast<const float*>(p.W0) + int64_t(ncol) * p.ldw
                                    : qkv_weight_row<float>(p, b_tile, ncol);
  for (int k0 = 0; k0 < p.K; k0 += FK) {
    int wcol = k0;
    if (MODE == kOut) {
      const int s = k0 / p.dh;
      wcol = head_of(p, b_tile, s) * p.dh + (k0 - s * p.dh);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      As[lk + e][lr] = a_row[k0 + lk + e];
      Bs[lk + e][lr] = w_row[wcol + lk + e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tr + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tc + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const RowMap om = map_row(p, tile_y, tr + i, FT);
    if (!om.valid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = n0 + tc + j;
      if (c < p.N) store_out<float, MODE>(p, om, c, acc[i][j]);
    }
  }
}

template <int MODE, int BMt, int BNt, int NW = 4>
int run_tile(GemmParams& p, const PrefillImp& pimp, hipStream_t stream, const char* name) {
  if (!p.seq_tiled && p.M_total >= (1 << 24)) p.seq_tiled = 1;
  int tiles_y;
  if (p.seq_tiled) {
    p.mt_per_seq = int(ceil_div(p.n, BMt));
    tiles_y = p.mt_per_seq * p.batch;
  } else {
    p.mt_per_seq = 0;
    tiles_y = int(ceil_div(p.M_total, BMt));
  }
  p.tiles_y = tiles_y;
  const int64_t total = ceil_div(p.N, BNt) * int64_t(tiles_y);
  const int64_t imp_blocks = MODE == kOut && pimp.pending ? int64_t(pimp.pieces) * pimp.batch : 0;
  const dim3 grid(unsigned(8 * ceil_div(total, 8) + imp_blocks));
  SPATTEN_TIMED(name, stream,
                (gemm_tile_kernel<MODE, BMt, BNt, NW><<<grid, 64 * NW, 0, stream>>>(p, pimp)));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

// Rounds of workgroups over the 256 CUs for a tile shape: tiles / (CUs x
// workgroups per CU), rounded up, since the last partial round costs a
// whole one.
inline double tile_rounds(const GemmParams& p, int bm, int bn, int per_cu) {
  const double my = p.seq_tiled ? double(ceil_div(p.n, bm)) * p.batch : double(ceil_div(p.M_total, bm));
  const double tiles = my * double(ceil_div(p.N, bn));
  return std::ceil(tiles / (256.0 * per_cu));
}

// pimp (output projection, optional): the prefill importance pass, carried
// by the tiled kernel's launch or run alone before the projection.
template <int MODE>
int run_gemm(GemmParams& p, int dtype, hipStream_t stream, const PrefillImp* pimp_in = nullptr) {
  PrefillImp pimp{};
  if (pimp_in) pimp = *pimp_in;
  const char* name = MODE == kOut ? "out_gemm" : "qkv_gemm";
  const int kt = skinny_kt(p.K);
  const bool skinny = MODE != kQkvPrefill && dtype == SPATTEN_BF16 && !p.seq_tiled &&
                      p.M_total <= 64 && p.N % 16 == 0 && kt > 0;
  const bool tiled = !skinny && dtype == SPATTEN_BF16 && MODE != kQkvDecode;
  if (pimp.pending && !tiled) {
    // only the tiled kernel carries the prefill importance pass
    const int st = launch_prefill_importance(pimp, stream);
    if (st != SPATTEN_OK) return st;
    pimp.pending = 0;
  }
  if (skinny) return run_skinny<MODE>(p, kt, stream, name);
  if (p.imp.pending) {
    // the projection takes a tiled path: the importance pass runs alone
    const int st = launch_importance(p.imp, stream);
    if (st != SPATTEN_OK) return st;
  }
  if (tiled) {
    // 128x128 tiles of four 64x64 waves run two workgroups per CU; 256x256
    // tiles of eight 128x64 waves run one, read a quarter fewer LDS bytes
    // per MFMA and finish a round in ~1.67x the time of a 128x128 round
    // (measured on MI355X: ~20% faster on 4096-deep projections). The
    // larger tile wins when its coarser rounds do not waste more than that.
    const double r128 = tile_rounds(p, 128, 128, 2), r256 = tile_rounds(p, 256, 256, 1);
    if (p.K >= 256 && 1.67 * r256 < 0.97 * r128)
      return run_tile<MODE, 256, 256, 8>(p, pimp, stream, name);
    return run_tile<MODE, 128, 128>(p, pimp, stream, name);
  }
  const int tm = dtype == SPATTEN_BF16 ? BM : FT;
  const int tn = dtype == SPATTEN_BF16 ? BN : FT;
  int tiles_y;
  if (p.seq_tiled) {
    p.mt_per_seq = int(ceil_div(p.n, tm));
    tiles_y = p.mt_per_seq * p.batch;
  } else {
    p.mt_per_seq = 0;
    tiles_y = int(ceil_div(p.M_total, tm));
  }
  const dim3 grid(unsigned(ceil_div(p.N, tn)), unsigned(tiles_y));
  if (dtype == SPATTEN_BF16)
    SPATTEN_TIMED(name, stream, gemm_bf16_kernel<MODE><<<grid, 256, 0, stream>>>(p));
  else
    SPATTEN_TIMED(name, stream, gemm_f32_kernel<MODE><<<grid, 256, 0, stream>>>(p));
  SPATTEN_LAUNCH_CHECK();
  return SPATTEN_OK;
}

}  // namespace

int launch_qkv(const QkvArgs& a, hipStream_t stream) {
  GemmParams p{};
  p.A = a.x;
  p.lda = a.D;
  p.W0 = a.w[0];
  p.W1 = a.w[1];
  p.W2 = a.w[2];
  p.ldw = a.D;
  p.head_idx = a.head_idx;
  p.batch = a.batch;
  p.n = a.n;
  // Tiles stay inside one sequence when heads differ per sequence, and for
  // prefill when n is not a multiple of 8: the V^T epilogue stores 8
  // consecutive rows of one sequence as one 16-byte chunk, which a tile
  // that starts mid-sequence would leave misaligned.
  p.seq_tiled = a.h_kept != a.D / a.dh || (a.mode == SPATTEN_PREFILL && a.n % 8 != 0);
  p.M_total = a.batch * a.n;
  p.N = 3 * a.h_kept * a.dh;
  p.K = a.D;
  p.h_kept = a.h_kept;
  p.dh = a.dh;
  p.D = a.D;
  p.n_pad = a.n_pad;
  p.out0 = a.q;
  p.out1 = a.k;
  p.out2 = a.vt;
  p.kv_bs = a.kv_bs;
  if (a.mode == SPATTEN_DECODE) return run_gemm<kQkvDecode>(p, a.dtype, stream);
  return run_gemm<kQkvPrefill>(p, a.dtype, stream);
}

int launch_out(const OutArgs& a, hipStream_t stream) {
  GemmParams p{};
  p.A = a.o;
  p.lda = int64_t(a.h_kept) * a.dh;
  p.W0 = a.wo;
  p.ldw = a.D;
  p.head_idx = a.head_idx;
  p.batch = a.batch;
  p.n = a.n;
  p.seq_tiled = a.h_kept != a.D / a.dh;
  p.M_total = a.batch * a.n;
  p.N = a.D;
  p.K = a.h_kept * a.dh;
  p.h_kept = a.h_kept;
  p.dh = a.dh;
  p.D = a.D;
  p.out0 = a.x;
  if (a.imp) p.imp = *a.imp;
  return run_gemm<kOut>(p, a.dtype, stream, a.pimp);
}

}  // namespace spatten
